// Host launchers of the measurement helpers in probes.hip (access-pattern read
// rates, agent-scope release costs), called by the ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {
// pattern 0..4, row_bytes a positive multiple of 256, bytes a positive multiple
// of the pattern's rows per region times row_bytes
bool read_pattern_shape_ok(int pattern, size_t bytes, size_t row_bytes);
hipError_t launch_read_pattern(int pattern, const void* src, size_t bytes, size_t row_bytes, int grid, uint32_t* sink,
                               hipStream_t s);
hipError_t launch_release_cost(int mode, float* data, uint32_t* ctr, int grid, int per_thread, hipStream_t s);
}  // namespace moe
