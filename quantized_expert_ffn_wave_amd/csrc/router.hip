// Router: logits = x Wr^T + b on the matrix cores, then top-k selection and
// routing weights with one wavefront per token.
//
// The review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", gives the selection
// structure: 6 of 256 routed experts per token.  The router form (a bf16
// Linear d_model -> experts, fp32 softmax, renormalised top-k) is the reading
// this library takes of that statement.
#include "common.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int ROUTER_KR = 256;                     // K range per split
constexpr int ROUTER_KS = D_MODEL / ROUTER_KR;     // 8 splits
constexpr int ROUTER_TG = 256;                     // tokens per workgroup

// Partial logits part[ks][t][e] = sum_{k in split ks} x[t][k] Wr[e][k].
// grid (ceil(E/64), ROUTER_KS, ceil(T/256)), 256 threads; wave w covers the
// 16 experts of tile 4*blockIdx.x + w and loops over the group's 16-token tiles.
// MFMA 16x16x32 bf16: A = x rows (tokens), B = Wr rows (experts), fp32 out.
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             float* __restrict__ part, int T, int E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = (blockIdx.x * 4 + wave) * 16;
  if (e0 >= E) return;
  const int ks = blockIdx.y;
  const int kbase = ks * ROUTER_KR + 8 * (lane >> 4);
  const int col = lane & 15;
  // B operand for all 8 k-steps of this split: 8 bf16 per step.
  bf16x8 b[ROUTER_KR / 32];
  const uint16_t* wrow = wr + (size_t)(e0 + col) * D_MODEL + kbase;
#pragma unroll
  for (int s = 0; s < ROUTER_KR / 32; ++s) b[s] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s);
  const int tg0 = blockIdx.z * ROUTER_TG;
  for (int t0 = tg0; t0 < min(T, tg0 + ROUTER_TG); t0 += 16) {
    const int t = t0 + col;
    bf16x8 a[ROUTER_KR / 32];
    if (t < T) {
      const uint16_t* xrow = x + (size_t)t * D_MODEL + kbase;
#pragma unroll
      for (int s = 0; s < ROUTER_KR / 32; ++s) a[s] = *reinterpret_cast<const bf16x8*>(xrow + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < ROUTER_KR / 32; ++s) a[s] = bf16x8{};
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < ROUTER_KR / 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
    // acc[j] = D[row 4*(lane/16)+j][col lane%16]: token t0 + 4*(lane>>4) + j, expert e0 + col
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 4 * (lane >> 4) + j;
      if (tt < T) part[((size_t)ks * T + tt) * E + e0 + col] = acc[j];
    }
  }
}

hipError_t launch_router(const LayerArgs& a, hipStream_t s) {
  dim3 grid((a.E + 63) / 64, ROUTER_KS, (a.T + ROUTER_TG - 1) / ROUTER_TG);
  hipLaunchKernelGGL(router_partial_kernel, grid, dim3(256), 0, s, a.x, a.router_w, a.logit_part, a.T, a.E);
  return hipGetLastError();
}

// Candidate order: a live candidate beats a dead one (taken, or no such
// expert); among live ones the larger logit wins, ties to the lower id.  NaN
// logits are ordered as -inf, so k distinct valid ids always come out.
__device__ inline bool better(bool al, float av, int ae, bool bl, float bv, int be) {
  if (al != bl) return al;
  return av > bv || (av == bv && ae < be);
}

// One wave per token: logit = sum of the 8 partials in split order (+ bias);
// k rounds of a wave-wide argmax; softmax weights.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                   float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, int T, int E, int K, int renorm,
                                                   int write_logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
  bool live[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    live[i] = e < E;
    v[i] = -INFINITY;
    if (live[i]) {
      float s = 0.f;
      for (int ks = 0; ks < ROUTER_KS; ++ks) s += part[((size_t)ks * T + t) * E + e];
      if (bias) s += bias[e];
      if (write_logits) logits[(size_t)t * E + e] = s;
      v[i] = (s != s) ? -INFINITY : s;
      mx = fmaxf(mx, v[i]);
    }
  }
  // wave max (for the all-experts softmax denominator)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float den_all = 0.f;
  if (!renorm) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (live[i]) den_all += expf(v[i] - mx);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den_all += __shfl_xor(den_all, off);
  }
  float sel_v[MAX_K];
  int sel_e[MAX_K];
#pragma unroll
  for (int j = 0; j < MAX_K; ++j) {
    sel_v[j] = -INFINITY;
    sel_e[j] = 0;
    if (j >= K) continue;
    // lane-local best (ids ascend with i, so ties keep the lower id)
    bool bl = live[0];
    float bv = v[0];
    int be = lane;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (better(live[i], v[i], lane + 64 * i, bl, bv, be)) { bl = live[i]; bv = v[i]; be = lane + 64 * i; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const bool ol = __shfl_xor((int)bl, off) != 0;
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (better(ol, ov, oe, bl, bv, be)) { bl = ol; bv = ov; be = oe; }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
    if ((be & 63) == lane) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == be) live[i] = false;
    }
  }
  if (lane < K) {
    float wv;
    int me = 0;
    float mv = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_K; ++j)
      if (j == lane) { me = sel_e[j]; mv = sel_v[j]; }
    if (renorm) {
      float den = 0.f;
#pragma unroll
      for (int j = 0; j < MAX_K; ++j)
        if (j < K) den += expf(sel_v[j] - sel_v[0]);
      wv = expf(mv - sel_v[0]) / den;
    } else {
      wv = expf(mv - mx) / den_all;
    }
    ids[(size_t)t * K + lane] = me;
    w[(size_t)t * K + lane] = wv;
  }
}

hipError_t launch_topk(const LayerArgs& a, bool write_logits, hipStream_t s) {
  dim3 grid((a.T + 3) / 4);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, s, a.logit_part, a.router_b, a.logits, a.ids, a.w, a.T, a.E,
                     a.K, a.renorm, write_logits ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
