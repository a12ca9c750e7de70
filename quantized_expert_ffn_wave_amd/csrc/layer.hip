// The layer's kernels in one translation unit: the routing and FFN device code,
// and the persistent decode kernel that calls both (device functions are not
// linked across translation units in this build).
#include "routing.hip"
#include "ffn.hip"
#include "decode.hip"
