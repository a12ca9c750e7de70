// Measurement helper, not part of the layer: the attainable rate of one kind
// of matrix-core instruction on this chip, to compare the tile path's
// matrix-core work with.  The NVFP4 files of the review ("What actually
// shipped", NVFP4 GGUF bullet) invite FP4-class instructions for prefill; this
// kernel shows what each instruction kind delivers when nothing else limits
// it.  Each wave keeps four independent accumulator chains (so that the
// instructions issue back to back rather than waiting on their own results)
// over operands held in registers, and writes the accumulators' sum at the
// end so that nothing is optimised away.
#include "common.hpp"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// kind 0: v_mfma_f32_32x32x16_f16; 1: _bf16; 2: _fp8_fp8 (E4M3 x E4M3);
// 3: v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 (E2M1) operands and unit E8M0 scales
template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* sink) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint32_t s = threadIdx.x * 0x9E3779B9u + blockIdx.x;  // operand bits that vary by lane
  const f16x8 ha = __builtin_bit_cast(f16x8, (u32x4){s & 0x3BFF3BFFu, s & 0x3BFF3BFFu, 0x3C003C00u, 0x3C003C00u});
  const bf16x8 ba = __builtin_bit_cast(bf16x8, (u32x4){s & 0x3F7F3F7Fu, 0x3F803F80u, s & 0x3F7F3F7Fu, 0x3F803F80u});
  const long fa = (long)(s & 0x3B3B3B3Bu) | ((long)(s & 0x3B3B3B3Bu) << 32);
  const i32x8 qa = {(int)(s & 0x77777777u), (int)(s & 0x77777777u), 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < iters; ++i) {
    if constexpr (KIND == 0) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, c3, 0, 0, 0);
    } else if constexpr (KIND == 1) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ba, ba, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ba, ba, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ba, ba, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ba, ba, c3, 0, 0, 0);
    } else if constexpr (KIND == 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa, fa, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa, fa, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa, fa, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa, fa, c3, 0, 0, 0);
    } else {
      // cbsz = blgp = 4: both operands FP4 E2M1; scale selectors 0, scales 0x7F (2^0)
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qa, c0, 4, 4, 0, 0x7F, 0, 0x7F);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qa, c1, 4, 4, 0, 0x7F, 0, 0x7F);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qa, c2, 4, 4, 0, 0x7F, 0, 0x7F);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, qa, c3, 4, 4, 0, 0x7F, 0, 0x7F);
    }
  }
  float v = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) v += (c0[k] + c1[k]) + (c2[k] + c3[k]);
  sink[(blockIdx.x * blockDim.x + threadIdx.x) & 255] = v;
}

hipError_t launch_mfma_rate(int kind, int iters, int grid, float* sink, hipStream_t s) {
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), dim3(256), 0, s, iters, sink); break;
    case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), dim3(256), 0, s, iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(grid), dim3(256), 0, s, iters, sink); break;
    default: hipLaunchKernelGGL(mfma_rate_kernel<3>, dim3(grid), dim3(256), 0, s, iters, sink); break;
  }
  return hipGetLastError();
}

}  // namespace moe
