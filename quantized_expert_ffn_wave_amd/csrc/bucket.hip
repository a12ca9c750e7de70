// Expert buckets: histogram of the chosen expert ids, exclusive prefix sum, a
// stable permutation of the slots (slot s = t*K + j) into expert-contiguous
// order, its inverse, and the FFN work lists.  One workgroup; deterministic.
//
// Stable ranks without atomics on the order: for a chunk of tokens, each slot
// sets bit (token) in its expert's LDS bitmask (OR is order independent); a
// slot's rank inside its bucket is then the number of set bits below its
// token, plus the bucket fill of earlier chunks.  A token has at most one slot
// per expert (its K ids are distinct), so ranks follow token order.
#include "common.hpp"

namespace moe {

constexpr int BK_THREADS = 1024;
constexpr int BK_TC = 1024;             // tokens per bitmask chunk
constexpr int BK_WORDS = BK_TC / 32;    // mask words per expert

// Items one expert contributes, per projection.
__device__ inline void expert_items(int m, int& nu, int& nd, int& tiles, bool& mfma) {
  if (m <= 0) { nu = nd = tiles = 0; mfma = false; return; }
  if (m <= GEMV_MAX) {
    mfma = false; tiles = 1;
    nu = D_FF / UP_GEMV_ROWS;
    nd = D_MODEL / DN_GEMV_ROWS;
  } else {
    mfma = true; tiles = (m + MFMA_BN - 1) / MFMA_BN;
    nu = tiles * (D_FF / UP_MFMA_ROWS);
    nd = tiles * (D_MODEL / DN_MFMA_ROWS);
  }
}

// Exclusive scan of v over n <= 320 entries by wave 0 (5 per lane); returns total.
__device__ int wave0_scan(int* v, int n) {
  const int lane = threadIdx.x & 63;
  int loc[5], sum = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int idx = lane * 5 + i;
    loc[i] = (idx < n) ? v[idx] : 0;
    sum += loc[i];
  }
  int inc = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  int run = inc - sum;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int idx = lane * 5 + i;
    if (idx < n) v[idx] = run;
    run += loc[i];
  }
  return __shfl(inc, 63);
}

__global__ __launch_bounds__(BK_THREADS) void bucket_kernel(LayerArgs a) {
  __shared__ int cnt[MAX_E + 1];
  __shared__ int off[MAX_E + 1];
  __shared__ int base[MAX_E];
  __shared__ uint32_t mask[MAX_E * BK_WORDS];
  __shared__ int it_mu[MAX_E + 2], it_md[MAX_E + 2], it_gu[MAX_E + 2], it_gd[MAX_E + 2];
  __shared__ int tot[4];
  const int tid = threadIdx.x;
  const int E = a.E, K = a.K, T = a.T, S = a.S;
  const int32_t* ids = a.ids;

  for (int e = tid; e < E; e += BK_THREADS) { cnt[e] = 0; base[e] = 0; }
  __syncthreads();
  for (int s = tid; s < S; s += BK_THREADS) atomicAdd(&cnt[ids[s]], 1);
  __syncthreads();
  if (tid < 64) {
    for (int e = tid; e < E; e += 64) off[e] = cnt[e];
    const int total = wave0_scan(off, E);
    if (tid == 0) off[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += BK_THREADS) a.counts[e] = cnt[e];
  for (int e = tid; e <= E; e += BK_THREADS) a.offsets[e] = off[e];

  // stable ranks, one token chunk at a time
  for (int t0 = 0; t0 < T; t0 += BK_TC) {
    for (int i = tid; i < E * BK_WORDS; i += BK_THREADS) mask[i] = 0u;
    __syncthreads();
    const int s0 = t0 * K, s1 = min(T, t0 + BK_TC) * K;
    for (int s = s0 + tid; s < s1; s += BK_THREADS) {
      const int tt = s / K - t0;
      atomicOr(&mask[ids[s] * BK_WORDS + (tt >> 5)], 1u << (tt & 31));
    }
    __syncthreads();
    for (int s = s0 + tid; s < s1; s += BK_THREADS) {
      const int e = ids[s], tt = s / K - t0;
      const uint32_t* me = mask + e * BK_WORDS;
      int r = base[e];
      for (int wd = 0; wd < (tt >> 5); ++wd) r += __popc(me[wd]);
      r += __popc(me[tt >> 5] & ((1u << (tt & 31)) - 1u));
      const int pos = off[e] + r;
      a.perm[pos] = s;
      a.inv_perm[s] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E; e += BK_THREADS) {
      int c = 0;
      for (int wd = 0; wd < BK_WORDS; ++wd) c += __popc(mask[e * BK_WORDS + wd]);
      base[e] += c;
    }
    __syncthreads();
  }

  // work lists: MFMA items first (heavier), then GEMV items; experts in order,
  // the shared expert (index E) last.
  const int NE = E + a.n_shared;
  for (int e = tid; e < NE; e += BK_THREADS) {
    const int m = (e < E) ? cnt[e] : T;
    int nu, nd, tiles;
    bool mf;
    expert_items(m, nu, nd, tiles, mf);
    it_mu[e] = mf ? nu : 0;
    it_md[e] = mf ? nd : 0;
    it_gu[e] = mf ? 0 : nu;
    it_gd[e] = mf ? 0 : nd;
  }
  __syncthreads();
  if (tid < 64) {
    const int a0 = wave0_scan(it_mu, NE);
    const int a1 = wave0_scan(it_md, NE);
    const int a2 = wave0_scan(it_gu, NE);
    const int a3 = wave0_scan(it_gd, NE);
    if (tid == 0) {
      it_mu[NE] = a0; it_md[NE] = a1; it_gu[NE] = a2; it_gd[NE] = a3;
      tot[0] = a0; tot[1] = a1; tot[2] = a2; tot[3] = a3;
    }
  }
  __syncthreads();
  const int n_up = min(tot[0] + tot[2], a.max_items_up);
  const int n_dn = min(tot[1] + tot[3], a.max_items_dn);
  if (tid == 0) {
    a.ctl[CTL_N_UP] = n_up;
    a.ctl[CTL_N_DN] = n_dn;
  }
  // fill both lists; item i -> expert by binary search over the item offsets
  for (int pass = 0; pass < 2; ++pass) {
    const int* mo = pass ? it_md : it_mu;
    const int* go = pass ? it_gd : it_gu;
    const int nm = pass ? tot[1] : tot[0];
    const int n = pass ? n_dn : n_up;
    uint32_t* out = pass ? a.items_dn : a.items_up;
    const int rows_m = pass ? (D_MODEL / DN_MFMA_ROWS) : (D_FF / UP_MFMA_ROWS);
    const int rows_g = pass ? (D_MODEL / DN_GEMV_ROWS) : (D_FF / UP_GEMV_ROWS);
    for (int i = tid; i < n; i += BK_THREADS) {
      const bool mf = i < nm;
      const int* o = mf ? mo : go;
      const int li = mf ? i : i - nm;
      int lo = 0, hi = NE;  // find e with o[e] <= li < o[e+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (o[mid] <= li) lo = mid; else hi = mid;
      }
      const int loc = li - o[lo];
      const int nch = mf ? rows_m : rows_g;
      out[i] = make_item(lo, loc % nch, loc / nch, mf);
    }
  }
}

hipError_t launch_bucket(const LayerArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(BK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
