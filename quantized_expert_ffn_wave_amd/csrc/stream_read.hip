// Plain streaming read of a device buffer: the attainable HBM read rate that
// the layer's weight streams are compared with.  Decoding with this layer is
// bound by moving expert weights from memory (orcarouter.ai review
// "Recursive Flint 40B-A2.5B", section "The architecture is an argument about
// memory bandwidth"); this kernel moves bytes and nothing else.
//
// Each thread keeps SR_DEPTH independent 16-byte nontemporal loads in flight
// per iteration over a grid-stride walk; the XOR of everything read decides a
// store that practically never happens, so that no load can be dropped.
#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int SR_THREADS = 256;
constexpr int SR_DEPTH = 8;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                  uint32_t* __restrict__ sink) {
  const size_t nth = (size_t)gridDim.x * SR_THREADS;
  size_t i = (size_t)blockIdx.x * SR_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (SR_DEPTH - 1) * nth < n16; i += SR_DEPTH * nth) {
    u32x4 v[SR_DEPTH];
#pragma unroll
    for (int d = 0; d < SR_DEPTH; ++d) v[d] = __builtin_nontemporal_load(p + i + d * nth);
#pragma unroll
    for (int d = 0; d < SR_DEPTH; ++d) acc ^= v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3];
  }
  for (; i < n16; i += nth) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // one lane-indexed slot per thread of the block: a vector store, never taken
  // for data that does not happen to XOR to this constant
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(SR_THREADS), 0, s, reinterpret_cast<const u32x4*>(src),
                     bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
