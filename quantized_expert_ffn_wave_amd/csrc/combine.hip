// Weighted combine of the expert outputs, and the residual/RMSNorm glue of the
// stacked layers.
//
// Per token: out = sum_j w_j * y[slot j] + shared_scale * y[shared], summed in
// the fixed order j = 0..K-1 then the shared expert, rounded once to bf16.  The
// review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", fixes the structure
// (6 routed experts plus one always-on shared expert per token, 47 MoE
// layers); the pre-norm residual form of the stack is this library's reading.
#include "common.hpp"

namespace moe {

constexpr int CB_THREADS = 256;
constexpr int CB_PER = D_MODEL / CB_THREADS;  // 8 elements per thread

__device__ inline void combine_row(const LayerArgs& a, int t, int i0, float* o) {
#pragma unroll
  for (int q = 0; q < CB_PER; ++q) o[q] = 0.f;
  for (int j = 0; j < a.K; ++j) {
    const float wj = a.w[(size_t)t * a.K + j];
    const int row = a.inv_perm[(size_t)t * a.K + j];
    const float4* p = reinterpret_cast<const float4*>(a.y + (size_t)row * D_MODEL + i0);
    const float4 v0 = p[0], v1 = p[1];
    o[0] += wj * v0.x; o[1] += wj * v0.y; o[2] += wj * v0.z; o[3] += wj * v0.w;
    o[4] += wj * v1.x; o[5] += wj * v1.y; o[6] += wj * v1.z; o[7] += wj * v1.w;
  }
  if (a.n_shared) {
    const float4* p = reinterpret_cast<const float4*>(a.y + (size_t)(a.S + t) * D_MODEL + i0);
    const float4 v0 = p[0], v1 = p[1];
    const float s = a.shared_scale;
    o[0] += s * v0.x; o[1] += s * v0.y; o[2] += s * v0.z; o[3] += s * v0.w;
    o[4] += s * v1.x; o[5] += s * v1.y; o[6] += s * v1.z; o[7] += s * v1.w;
  }
}

__device__ inline void store_bf16x8(uint16_t* dst, const float* v) {
  uint4 pk;
  pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  pk.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
  pk.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  *reinterpret_cast<uint4*>(dst) = pk;
}

__global__ __launch_bounds__(CB_THREADS) void combine_kernel(LayerArgs a, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int i0 = CB_PER * threadIdx.x;
  float o[CB_PER];
  combine_row(a, t, i0, o);
  store_bf16x8(out + (size_t)t * D_MODEL + i0, o);
}

hipError_t launch_combine(const LayerArgs& a, uint16_t* out, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(CB_THREADS), 0, s, a, out);
  return hipGetLastError();
}

// Sum of v over the workgroup (all threads receive it).
__device__ inline float block_sum(float v) {
  __shared__ float part[CB_THREADS / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CB_THREADS / 64; ++i) s += part[i];
  return s;
}

// xn = bf16(r / sqrt(mean(r^2) + eps)) for the 8 values of this thread.
__device__ inline void rmsnorm_store(const float* r, uint16_t* xn_row, int i0, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < CB_PER; ++q) ss += r[q] * r[q];
  ss = block_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D_MODEL + eps);
  float v[CB_PER];
#pragma unroll
  for (int q = 0; q < CB_PER; ++q) v[q] = r[q] * inv;
  store_bf16x8(xn_row + i0, v);
}

// r = x (bf16 -> fp32); xn = bf16(RMSNorm(r)).
__global__ __launch_bounds__(CB_THREADS) void stack_init_kernel(const uint16_t* __restrict__ x, float* __restrict__ r,
                                                                uint16_t* __restrict__ xn, float eps) {
  const int t = blockIdx.x;
  const int i0 = CB_PER * threadIdx.x;
  const uint4 pk = *reinterpret_cast<const uint4*>(x + (size_t)t * D_MODEL + i0);
  const uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
  float v[CB_PER];
#pragma unroll
  for (int q = 0; q < 4; ++q) { v[2 * q] = __uint_as_float(w[q] << 16); v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u); }
  float4* rp = reinterpret_cast<float4*>(r + (size_t)t * D_MODEL + i0);
  rp[0] = make_float4(v[0], v[1], v[2], v[3]);
  rp[1] = make_float4(v[4], v[5], v[6], v[7]);
  rmsnorm_store(v, xn + (size_t)t * D_MODEL, i0, eps);
}

hipError_t launch_stack_init(const uint16_t* x, float* r, uint16_t* xn, int T, float eps, hipStream_t s) {
  hipLaunchKernelGGL(stack_init_kernel, dim3(T), dim3(CB_THREADS), 0, s, x, r, xn, eps);
  return hipGetLastError();
}

// Layer output y = bf16(combine); r += y; then either the next layer's input
// xn = bf16(RMSNorm(r)) or, after the last layer, x_final = bf16(r).
// y_rec (optional) receives the layer output.
__global__ __launch_bounds__(CB_THREADS) void combine_stack_kernel(LayerArgs a, float* __restrict__ r,
                                                                   uint16_t* __restrict__ xn_next,
                                                                   uint16_t* __restrict__ y_rec,
                                                                   uint16_t* __restrict__ x_final, float eps) {
  const int t = blockIdx.x;
  const int i0 = CB_PER * threadIdx.x;
  float o[CB_PER];
  combine_row(a, t, i0, o);
  float yb[CB_PER];
#pragma unroll
  for (int q = 0; q < CB_PER; ++q) yb[q] = bf16_to_f32(f32_to_bf16(o[q]));
  if (y_rec) store_bf16x8(y_rec + (size_t)t * D_MODEL + i0, yb);
  float4* rp = reinterpret_cast<float4*>(r + (size_t)t * D_MODEL + i0);
  const float4 r0 = rp[0], r1 = rp[1];
  float rv[CB_PER] = {r0.x + yb[0], r0.y + yb[1], r0.z + yb[2], r0.w + yb[3],
                      r1.x + yb[4], r1.y + yb[5], r1.z + yb[6], r1.w + yb[7]};
  rp[0] = make_float4(rv[0], rv[1], rv[2], rv[3]);
  rp[1] = make_float4(rv[4], rv[5], rv[6], rv[7]);
  if (x_final) store_bf16x8(x_final + (size_t)t * D_MODEL + i0, rv);
  if (xn_next) rmsnorm_store(rv, xn_next + (size_t)t * D_MODEL, i0, eps);
}

hipError_t launch_combine_stack(const LayerArgs& a, float* r, uint16_t* xn_next, uint16_t* y_rec, uint16_t* x_final,
                                float eps, hipStream_t s) {
  hipLaunchKernelGGL(combine_stack_kernel, dim3(a.T), dim3(CB_THREADS), 0, s, a, r, xn_next, y_rec, x_final, eps);
  return hipGetLastError();
}

}  // namespace moe
