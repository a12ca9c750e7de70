// Routing: router logits on the matrix cores, top-k selection with softmax
// weights (one wavefront per token), and the expert buckets and work lists.
//
// The review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", gives the selection
// structure: 6 of 256 routed experts per token plus an always-on shared
// expert.  The router form (bf16 Linear d_model -> experts, fp32 softmax over
// the chosen experts) is this library's reading of that statement.
//
// Kernel boundaries order the steps (no device-scope fences):
//   router        partial logits part[ks][t][e] over 8 K-splits, or 4 beyond 256
//                 tokens (MFMA 16x16x32 bf16);
//   topk          one wave per token sums the partials in split order, selects
//                 the top k (ties to the lower id: wave-wide maxima of 32-bit
//                 order-preserving keys with permlane swaps and DPP, then a
//                 ballot) and writes the weights;
//   bucket        histogram, exclusive prefix sum, a stable slot permutation from
//                 per-expert token bitmasks and popcounts, its inverse, and the
//                 FFN work lists: one workgroup up to 256 tokens, else three
//                 launches over 256-token chunks.
#include "common.hpp"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int ROUTER_KR = 256;                  // K range per split (T <= ROUTER_SMALL_T)
constexpr int ROUTER_KS = D_MODEL / ROUTER_KR;  // 8 splits
constexpr int ROUTER_SMALL_T = 256;             // largest T for one 16-token tile per wave
constexpr int ROUTER_KS_L = 4;                  // K-splits for larger T
constexpr int ROUTER_KR_L = D_MODEL / ROUTER_KS_L;
constexpr int ROUTER_TG = 64;                   // tokens per workgroup for larger T
constexpr int ROUTER_XS = ROUTER_KR_L + 8;      // LDS row stride of the staged activations
// partial logit splits the top-k sums for a batch of T tokens
__host__ __device__ inline int router_splits(int T) { return T <= ROUTER_SMALL_T ? ROUTER_KS : ROUTER_KS_L; }

// Decode-sized T: one wave per (16-token tile, 16-expert tile, K-split); the
// workgroup's 4 waves take 4 consecutive expert tiles.  grid (ceil(T/16) *
// ceil(E/64), ROUTER_KS).  MFMA 16x16x32 bf16: A = x rows, B = router rows.
// (bx, ks): the workgroup's (token tile x expert group, K-split) indices
__device__ inline void router_small_tile(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                         const float* __restrict__ bias, float* __restrict__ part, int T, int E,
                                         int bx, int ks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int egroups = (E + 63) / 64;
  const int t0 = (bx / egroups) * 16;
  const int e0 = ((bx % egroups) * 4 + wave) * 16;
  if (e0 >= E) return;
  const int kbase = ks * ROUTER_KR + 8 * (lane >> 4);
  const int col = lane & 15;
  const int t = t0 + col;
  bf16x8 a[ROUTER_KR / 32], b[ROUTER_KR / 32];
  const uint16_t* wrow = wr + (size_t)(e0 + col) * D_MODEL + kbase;
  const uint16_t* xrow = x + (size_t)(t < T ? t : 0) * D_MODEL + kbase;
#pragma unroll
  for (int s = 0; s < ROUTER_KR / 32; ++s) {
    b[s] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s);
    a[s] = (t < T) ? *reinterpret_cast<const bf16x8*>(xrow + 32 * s) : bf16x8{};
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < ROUTER_KR / 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
  // acc[j] = D[row 4*(lane/16)+j][col lane%16]: token t0 + 4*(lane>>4) + j, expert e0 + col
  const float bz = (ks == 0 && bias) ? bias[e0 + col] : 0.f;  // the bias rides in split 0
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tt = t0 + 4 * (lane >> 4) + j;
    if (tt < T) part[((size_t)ks * T + tt) * E + e0 + col] = acc[j] + bz;
  }
}

__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, float* __restrict__ part,
                                                           int T, int E) {
  router_small_tile(x, wr, bias, part, T, E, blockIdx.x, blockIdx.y);
}

// Larger T: one 1024-thread workgroup per (64-token group, K-split of 512).
// Wave w keeps router rows 16 w .. 16 w + 15 of the split in registers, so the
// 16 waves cover 256 experts, and the 16-token activation tiles are staged once
// in LDS for all of them (double buffered, one barrier per tile): the
// activations are read once, not once per group of experts.
// grid (ceil(T/ROUTER_TG), ROUTER_KS_L).
__global__ __launch_bounds__(1024) void router_large_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias, float* __restrict__ part,
                                                            int T, int E) {
  __shared__ uint16_t xs[2][16 * ROUTER_XS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = blockIdx.y, k0 = ks * ROUTER_KR_L;
  const int col = lane & 15, kq = lane >> 4;
  const int e = 16 * wave + col;  // this lane's expert (B column / output column)
  const bool ev = e < E;
  bf16x8 b[ROUTER_KR_L / 32];
  const uint16_t* wrow = wr + (size_t)(ev ? e : 0) * D_MODEL + k0 + 8 * kq;
#pragma unroll
  for (int s = 0; s < ROUTER_KR_L / 32; ++s) b[s] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s);
  const float bz = (ks == 0 && bias && ev) ? bias[e] : 0.f;  // the bias rides in split 0
  const int tg0 = blockIdx.x * ROUTER_TG, tg1 = min(T, tg0 + ROUTER_TG);
  // staging: thread tid holds 8 activations (16 B) of row tid / 64 of a tile
  const int sr = tid >> 6, sc = 8 * (tid & 63);
  auto stage_load = [&](int t0) {
    return *reinterpret_cast<const bf16x8*>(x + (size_t)min(t0 + sr, T - 1) * D_MODEL + k0 + sc);
  };
  bf16x8 v = stage_load(tg0);
  int buf = 0;
  for (int t0 = tg0; t0 < tg1; t0 += 16) {
    *reinterpret_cast<bf16x8*>(&xs[buf][sr * ROUTER_XS + sc]) = v;
    __syncthreads();
    v = stage_load(min(t0 + 16, tg1 - 1));  // always issued; the last one is not stored
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < ROUTER_KR_L / 32; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&xs[buf][col * ROUTER_XS + 32 * s + 8 * kq]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[s], acc, 0, 0, 0);
    }
    // acc[j] = token t0 + 4 kq + j, expert e
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = t0 + 4 * kq + j;
      if (tt < tg1 && ev) part[((size_t)ks * T + tt) * E + e] = acc[j] + bz;
    }
    buf ^= 1;
  }
}

hipError_t launch_router(const LayerArgs& a, hipStream_t s) {
  if (a.T <= ROUTER_SMALL_T) {
    dim3 grid(ceil_div(a.T, 16) * ceil_div(a.E, 64), ROUTER_KS);
    hipLaunchKernelGGL(router_small_kernel, grid, dim3(256), 0, s, a.x, a.router_w, a.router_b, a.logit_part, a.T, a.E);
  } else {
    dim3 grid(ceil_div(a.T, ROUTER_TG), ROUTER_KS_L);
    hipLaunchKernelGGL(router_large_kernel, grid, dim3(1024), 0, s, a.x, a.router_w, a.router_b, a.logit_part, a.T,
                       a.E);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// top-k + buckets
// ---------------------------------------------------------------------------------------
constexpr int TK_THREADS = 256;             // 4 waves: 4 tokens per workgroup
constexpr int BK_THREADS = 1024;

// Selection key: the order-preserving bits of a logit (NaN ordered as -inf,
// -0 as +0); equal keys go to the lower expert id.
__device__ inline uint32_t ordered_bits(float v) {
  if (v != v) v = -INFINITY;
  if (v == 0.f) v = 0.f;  // -0 and +0 are one value
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// One wave: logits of token t (sum of the KS partials in split order + bias),
// the top k ids and their weights.
template <int KS>
__device__ void topk_token(const LayerArgs& a, int t, int32_t* lds_ids) {
  const int lane = threadIdx.x & 63;
  const int T = a.T, E = a.E, K = a.K;
  // all 8 x 4 partial sums in flight at once (lanes past E read a valid
  // entry and are masked below); the bias is already in split 0
  float p[4][KS];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = min(lane + 64 * i, E - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) p[i][ks] = a.logit_part[((size_t)ks * T + t) * E + e];
  }
  // 4-bit formats: the token's activation scale for the fp16 operands of the
  // expert products, from the largest |x| of its row (32 elements per lane),
  // and the row scaled into fp16 for the matrix-core tiles, in the weights' k
  // order: natural for NVFP4; for q4_1, within each group of 8 elements the
  // order 0 4 1 5 2 6 3 7 in which its nibble decode delivers the weights
  if (a.fmt != FMT_BF16) {
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)t * D_MODEL) + 4 * lane;
    uint4 xv[4];
    uint32_t mx = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = xr[i];
      const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) mx = max(mx, max(w4[q] & 0x7FFFu, (w4[q] >> 16) & 0x7FFFu));
    }
    mx = wave_max_u32(mx);
    const float sc = pow2_scale(mx << 16);
    if (lane == 0) a.xsc[t] = sc;
    if (a.xq != nullptr) {  // (none where the batch has no tile)
      uint4* dst = reinterpret_cast<uint4*>(a.xq + (size_t)t * D_MODEL) + 4 * lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        uint32_t n[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          n[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w4[q] << 16) * sc,
                                                                       __uint_as_float(w4[q] & 0xFFFF0000u) * sc));
        if (a.fmt == FMT_Q4_1)
          dst[i] = make_uint4(__builtin_amdgcn_perm(n[2], n[0], 0x05040100u), __builtin_amdgcn_perm(n[2], n[0], 0x07060302u),
                              __builtin_amdgcn_perm(n[3], n[1], 0x05040100u), __builtin_amdgcn_perm(n[3], n[1], 0x07060302u));
        else dst[i] = make_uint4(n[0], n[1], n[2], n[3]);
      }
    }
  }
  uint32_t kk[4];
  float mx = -INFINITY;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s += p[i][ks];
    kk[i] = 0u;
    v[i] = -INFINITY;
    if (e < E) {
      if (a.write_logits) a.logits[(size_t)t * E + e] = s;
      v[i] = (s != s) ? -INFINITY : s;
      kk[i] = ordered_bits(s);
      mx = fmaxf(mx, v[i]);
    }
  }
  float den_all = 0.f;
  if (!a.renorm) {
    mx = from_ordered(wave_max_u32(ordered_bits(mx)));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i < E) den_all += expf(v[i] - mx);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den_all += __shfl_xor(den_all, off);
  }
  // K rounds: the wave-wide maximum of the 32-bit order-preserving keys, then
  // the lowest expert id holding it (a ballot per group of 64 ids), which is
  // taken out.  Key 0 marks a taken or missing expert (every logit, -inf and
  // NaN included, has a larger key).
  float sel_v[MAX_K];
  int sel_e[MAX_K];
#pragma unroll
  for (int j = 0; j < MAX_K; ++j) {
    sel_v[j] = -INFINITY;
    sel_e[j] = 0;
    if (j >= K) continue;
    const uint32_t m = wave_max_u32(max(max(kk[0], kk[1]), max(kk[2], kk[3])));
    uint64_t bal = __ballot(kk[0] == m);
    int e = 0;
    if (bal) {
      e = __builtin_ctzll(bal);
    } else if ((bal = __ballot(kk[1] == m))) {
      e = 64 + __builtin_ctzll(bal);
    } else if ((bal = __ballot(kk[2] == m))) {
      e = 128 + __builtin_ctzll(bal);
    } else {
      e = 192 + __builtin_ctzll(__ballot(kk[3] == m));
    }
    sel_e[j] = e;
    sel_v[j] = from_ordered(m);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == e) kk[i] = 0u;
  }
  if (lane < K) {
    float wv;
    int me = 0;
    float mv = 0.f;
#pragma unroll
    for (int j = 0; j < MAX_K; ++j)
      if (j == lane) { me = sel_e[j]; mv = sel_v[j]; }
    if (a.renorm) {
      float den = 0.f;
#pragma unroll
      for (int j = 0; j < MAX_K; ++j)
        if (j < K) den += expf(sel_v[j] - sel_v[0]);
      wv = expf(mv - sel_v[0]) / den;
    } else {
      wv = expf(mv - mx) / den_all;
    }
    a.ids[(size_t)t * K + lane] = me;
    a.w[(size_t)t * K + lane] = wv;
    if (lds_ids) lds_ids[t * K + lane] = me;
  }
}

// Exclusive scan of v over n <= 320 entries by one wave (5 per lane); returns total.
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

struct ListSmem {
  int it_m[MAX_E + 2];   // matrix-core tiles per expert, then their exclusive prefix
  int it_g[MAX_E + 2];   // vector tiles per expert, then their exclusive prefix
  int tot[2];
};


// Work lists from the bucket sizes cnt[e] and offsets off[e] (in LDS);
// perm_at(p) gives the slot at bucket position p.
template <typename PermAt>
__device__ void write_lists(const LayerArgs& a, const int* bcnt, const int* boff, ListSmem& ls, PermAt perm_at) {
  const int tid = threadIdx.x, nth = blockDim.x;
  const int E = a.E, K = a.K, T = a.T;
  // work list: matrix-core tiles first, then vector tiles.  A matrix-core tile
  // makes mf_up_chunks(bn) gate/up items and N_DN_CHUNKS down items, a vector tile
  // vec_up_chunks(T) and vec_dn_chunks(T); item i of a kind is chunk i % chunks of its
  // tile i / chunks (vector items counted from the first vector tile).
  const int bn = mfma_bn(T);
  for (int e = tid; e < E; e += nth) {
    const int m = bcnt[e];
    const int tiles = bucket_tiles(m, T);
    ls.it_m[e] = bucket_mfma(m, T) ? tiles : 0;
    ls.it_g[e] = bucket_mfma(m, T) ? 0 : tiles;
  }
  __syncthreads();
  if (tid < 64) {
    const int a0 = wave0_scan(ls.it_m, E);
    if (tid == 0) ls.it_m[E] = ls.tot[0] = a0;
  } else if (tid < 128) {
    const int a1 = wave0_scan(ls.it_g, E);
    if (tid == 64) ls.it_g[E] = ls.tot[1] = a1;
  }
  __syncthreads();
  const int tiles_m = ls.tot[0], tiles_g = ls.tot[1];
  // The shared expert takes every token: bn-token matrix-core tiles from
  // mfma_min(T) tokens on, else groups of GV_GROUP tokens, in the same lists.
  // Tile order: routed matrix-core, shared matrix-core, shared vector, routed
  // vector (the kernels take the matrix-core items first; the shared expert's
  // vector items, which mostly read its weights from L2, go before the routed
  // ones so that they do not fall into the last, partial round).
  const int sh_tiles = a.n_shared ? shared_tiles(T) : 0;
  const bool sh_mf = shared_mfma(T);
  const int mf_tiles = tiles_m + (sh_mf ? sh_tiles : 0);
  const int sh_vec = sh_mf ? 0 : sh_tiles;
  const int all_tiles = tiles_m + tiles_g + sh_tiles;
  const int n_tiles = min(all_tiles, a.max_tiles);
  // (batches with matrix-core tiles have the standard vector items)
  const int n_up = n_tiles * vec_up_chunks(T), n_dn = n_tiles * vec_dn_chunks(T);
  if (tid == 0) {
    a.ctl[CTL_N_UP] = n_up;
    a.ctl[CTL_N_DN] = n_dn;
    a.ctl[CTL_N_UP_MF] = min(mf_tiles, n_tiles) * mf_up_chunks(bn);
    a.ctl[CTL_N_DN_MF] = min(mf_tiles, n_tiles) * N_DN_CHUNKS;
  }
  // one thread per token tile: its entry (row chunk 0; the kernels derive the
  // chunk from the item index)
  for (int ti = tid; ti < n_tiles; ti += nth) {
    const bool shared = (ti >= tiles_m && ti < mf_tiles + sh_vec);
    const bool mf = ti < mf_tiles;
    const int per = mf ? bn : GV_GROUP;
    int expert, p0, cnt;
    uint32_t tk[GV_GROUP] = {0u, 0u, 0u, 0u};
    if (shared) {
      const int tile = mf ? ti - tiles_m : ti - mf_tiles;
      expert = SHARED_ID;
      p0 = tile * per;
      cnt = min(per, T - p0);
      for (int j = 0; j < cnt && j < GV_GROUP; ++j) tk[j] = (uint32_t)(p0 + j);
    } else {
      const int* o = mf ? ls.it_m : ls.it_g;
      const int li = mf ? ti : ti - mf_tiles - sh_vec;
      int lo = 0, hi = E;  // the expert e with o[e] <= li < o[e+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (o[mid] <= li) lo = mid; else hi = mid;
      }
      const int tile = li - o[lo];
      expert = lo;
      p0 = boff[lo] + tile * per;
      cnt = min(per, bcnt[lo] - tile * per);
      if (!mf) {
        for (int j = 0; j < cnt; ++j) tk[j] = (uint32_t)(perm_at(p0 + j) / K);
      }
    }
    Item it;
    it.head = item_head(expert, 0, cnt, mf);
    it.p0 = (uint32_t)p0;
    it.t01 = tk[0] | (tk[1] << 16);
    it.t23 = tk[2] | (tk[3] << 16);
    a.tiles[ti] = it;
  }
}

// KS: the router's partial splits for this batch size (router_splits(T))
template <int KS>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(LayerArgs a) {
  const int t = blockIdx.x * (TK_THREADS / 64) + (threadIdx.x >> 6);
  if (t < a.T) topk_token<KS>(a, t, nullptr);
}

// ---------------------------------------------------------------------------------------
// Large batches (T > RS_MAX_T): buckets in chunks of BK_CT tokens, three launches.
//   chunk_hist   one workgroup per chunk: slots per expert in the chunk;
//   chunk_scan   one workgroup: bucket sizes and offsets, each chunk's first
//                position in every bucket, and the work lists (vector-path
//                items without their token ids);
//   chunk_perm   one workgroup per chunk: a slot's rank among the chunk's slots
//                of its expert (token bitmasks and popcounts), hence its bucket
//                position, the permutation and its inverse, and the token ids of
//                the vector-path items.
// The partial-logit region, consumed by the top-k, holds the chunk table
// base[chunk][e] and, after it, each expert's first vector-path tile (or -1).
// ---------------------------------------------------------------------------------------
constexpr int BK_CT = 256;
constexpr int BK_CW = BK_CT / 32;

__device__ inline int32_t* chunk_table(const LayerArgs& a) { return reinterpret_cast<int32_t*>(a.logit_part); }

__global__ __launch_bounds__(BK_THREADS) void chunk_hist_kernel(LayerArgs a) {
  __shared__ int cnt[MAX_E];
  const int tid = threadIdx.x, E = a.E, K = a.K;
  const int t0 = blockIdx.x * BK_CT, t1 = min(a.T, t0 + BK_CT);
  for (int e = tid; e < E; e += BK_THREADS) cnt[e] = 0;
  __syncthreads();
  for (int s = t0 * K + tid; s < t1 * K; s += BK_THREADS) atomicAdd(&cnt[a.ids[s]], 1);
  __syncthreads();
  int32_t* base = chunk_table(a) + (size_t)blockIdx.x * E;
  for (int e = tid; e < E; e += BK_THREADS) base[e] = cnt[e];
}

__global__ __launch_bounds__(BK_THREADS) void chunk_scan_kernel(LayerArgs a) {
  __shared__ int cnt[MAX_E + 1];
  __shared__ int off[MAX_E + 1];
  __shared__ ListSmem ls;
  const int tid = threadIdx.x, E = a.E;
  const int nch = ceil_div(a.T, BK_CT);
  int32_t* tab = chunk_table(a);
  // per expert: exclusive running sum over the chunks (in place), then the total
  for (int e = tid; e < E; e += BK_THREADS) {
    int run = 0;
    for (int c0 = 0; c0 < nch; c0 += 8) {
      int h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (c0 + i < nch) ? tab[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c0 + i < nch) tab[(size_t)(c0 + i) * E + e] = run;
        run += h[i];
      }
    }
    cnt[e] = off[e] = run;
  }
  __syncthreads();
  if (tid < 64) {
    const int total = wave0_scan(off, E);
    if (tid == 0) off[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += BK_THREADS) a.counts[e] = cnt[e];
  for (int e = tid; e <= E; e += BK_THREADS) a.offsets[e] = off[e];
  for (int i = tid; i < nch * E; i += BK_THREADS) tab[i] += off[i % E];
  write_lists(a, cnt, off, ls, [](int) { return 0; });
  // first vector-path tile of each expert (tile order: routed matrix-core,
  // shared matrix-core, shared vector, routed vector)
  const int sh_all = a.n_shared ? shared_tiles(a.T) : 0;  // matrix-core or vector, first either way
  int32_t* vt = tab + (size_t)nch * E;
  for (int e = tid; e < E; e += BK_THREADS)
    vt[e] = bucket_mfma(cnt[e], a.T) ? -1 : ls.tot[0] + sh_all + ls.it_g[e];
}

__global__ __launch_bounds__(BK_THREADS) void chunk_perm_kernel(LayerArgs a) {
  __shared__ int32_t ids[BK_CT * MAX_K];
  __shared__ uint32_t mask[MAX_E * BK_CW];
  const int tid = threadIdx.x, E = a.E, K = a.K;
  const int t0 = blockIdx.x * BK_CT, t1 = min(a.T, t0 + BK_CT);
  const int s0 = t0 * K, ns = (t1 - t0) * K;
  const int nch = ceil_div(a.T, BK_CT);
  const int32_t* base = chunk_table(a) + (size_t)blockIdx.x * E;
  const int32_t* vt = chunk_table(a) + (size_t)nch * E;
  const int n_tiles = a.ctl[CTL_N_UP] / N_UP_CHUNKS;
  for (int i = tid; i < ns; i += BK_THREADS) ids[i] = a.ids[s0 + i];
  for (int i = tid; i < E * BK_CW; i += BK_THREADS) mask[i] = 0u;
  __syncthreads();
  for (int i = tid; i < ns; i += BK_THREADS) {
    const int tt = i / K;
    atomicOr(&mask[ids[i] * BK_CW + (tt >> 5)], 1u << (tt & 31));
  }
  __syncthreads();
  for (int i = tid; i < ns; i += BK_THREADS) {
    const int e = ids[i], tt = i / K;
    const uint32_t* me = mask + e * BK_CW;
    int r = 0;
    for (int w = 0; w < (tt >> 5); ++w) r += __popc(me[w]);
    r += __popc(me[tt >> 5] & ((1u << (tt & 31)) - 1u));
    const int pos = base[e] + r;
    a.perm[pos] = s0 + i;
    a.inv_perm[s0 + i] = pos;
    if (vt[e] >= 0) {  // a vector-path bucket: the token's id goes into its item
      const int g = pos - a.offsets[e];
      const int ti = vt[e] + g / GV_GROUP;
      if (ti < n_tiles) reinterpret_cast<uint16_t*>(a.tiles + ti)[4 + g % GV_GROUP] = (uint16_t)(t0 + tt);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Decode-sized batches (T <= RS_MAX_T): buckets and work lists in one
// workgroup with the ids, token masks and the permutation in LDS.  Up to
// RS_FUSED_T tokens (one per wave) the same workgroup also runs the top-k.
// ---------------------------------------------------------------------------------------
constexpr int RS_THREADS = 1024;
constexpr int RS_MAX_T = 256;
constexpr int RS_FUSED_T = RS_THREADS / 64;
constexpr int RS_WORDS = RS_MAX_T / 32;

struct RouteSmallSmem {
  int32_t ids[RS_MAX_T * MAX_K];
  uint32_t mask[MAX_E * RS_WORDS];
  int off[MAX_E + 1];    // bucket offsets (exclusive prefix of the sizes)
  int it_m[MAX_E];       // first routed matrix-core tile of each expert
  int vt[MAX_E];         // its first vector tile (an index into the list), or -1
  int wtot[4][3];        // per wave of experts: sizes, matrix-core tiles, vector tiles
};

// Tile i of the shared expert, which takes every token: bn-token matrix-core
// tiles (mf), or groups of GV_GROUP tokens with their ids.
__device__ inline Item shared_tile(int T, int i, bool mf, int bn) {
  const int per = mf ? bn : GV_GROUP;
  const int p0 = i * per, cnt = min(per, T - p0);
  uint32_t tk[GV_GROUP] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < GV_GROUP; ++j)
    if (!mf && j < cnt) tk[j] = (uint32_t)(p0 + j);
  Item it;
  it.head = item_head(SHARED_ID, 0, cnt, mf);
  it.p0 = (uint32_t)p0;
  it.t01 = tk[0] | (tk[1] << 16);
  it.t23 = tk[2] | (tk[3] << 16);
  return it;
}

// inclusive prefix sum over the wave's lanes
__device__ inline int wave_inclusive(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Buckets and work lists of T <= RS_MAX_T tokens in one 1024-thread
// workgroup, in four barrier-separated phases: ids into LDS (TOPK: the
// workgroup runs the top-k itself, one wave per token); per-expert token
// bitmasks; per expert (one thread each, E <= 256) its bucket size and tile
// counts, prefix-summed within each wave and then across the four waves; and
// the outputs: the bucket sizes and offsets, the stable slot permutation and
// its inverse (a slot's rank r in its bucket = tokens of that expert before
// it), and the tile entries: a slot of a vector-path bucket writes its token
// id into tile r / 4 (and slot 4 k the tile's head), each expert its
// matrix-core tiles, and the threads past the experts the shared expert's
// tiles.  Tile order: routed
// matrix-core, shared matrix-core, shared vector, routed vector (the kernels
// take the matrix-core items first; the shared expert's vector items, which
// mostly read its weights from L2, go before the routed ones so that they do
// not fall into the last, partial round).
template <bool TOPK>
__device__ void route_small(const LayerArgs& a, RouteSmallSmem& sm) {
  const int tid = threadIdx.x, nth = blockDim.x, wave = tid >> 6, lane = tid & 63;
  const int E = a.E, K = a.K, T = a.T, S = a.S;
  const int W = ceil_div(T, 32);
  if (TOPK) {
    for (int t = wave; t < T; t += nth / 64) topk_token<ROUTER_KS>(a, t, sm.ids);
  } else {
    for (int s = tid; s < S; s += nth) sm.ids[s] = a.ids[s];
  }
  for (int i = tid; i < E * W; i += nth) sm.mask[i] = 0u;
  __syncthreads();
  // per-expert token masks (a token holds at most one slot of an expert)
  for (int s = tid; s < S; s += nth) {
    const int t = s / K;
    atomicOr(&sm.mask[sm.ids[s] * W + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  // thread e < E: bucket size and tiles, prefix sums within its wave
  const int bn = mfma_bn(T);
  int c = 0, tm = 0, tg = 0, c_in = 0, tm_in = 0, tg_in = 0;
  if (wave < 4) {
    if (tid < E) {
      for (int w = 0; w < W; ++w) c += __popc(sm.mask[tid * W + w]);
      const int tiles = bucket_tiles(c, T);
      tm = bucket_mfma(c, T) ? tiles : 0;
      tg = bucket_mfma(c, T) ? 0 : tiles;
    }
    c_in = wave_inclusive(c);
    tm_in = wave_inclusive(tm);
    tg_in = wave_inclusive(tg);
    if (lane == 63) {
      sm.wtot[wave][0] = c_in;
      sm.wtot[wave][1] = tm_in;
      sm.wtot[wave][2] = tg_in;
    }
  }
  __syncthreads();
  // totals over the waves of experts, and each expert's exclusive prefixes
  int tot_c = 0, tiles_m = 0, tiles_g = 0, pre_c = 0, pre_m = 0, pre_g = 0;
  for (int v = 0; v < 4; ++v) {
    if (v < wave) {
      pre_c += sm.wtot[v][0];
      pre_m += sm.wtot[v][1];
      pre_g += sm.wtot[v][2];
    }
    tot_c += sm.wtot[v][0];
    tiles_m += sm.wtot[v][1];
    tiles_g += sm.wtot[v][2];
  }
  const int sh_tiles = a.n_shared ? shared_tiles(T) : 0;
  const bool sh_mf = shared_mfma(T);
  const int mf_tiles = tiles_m + (sh_mf ? sh_tiles : 0);
  const int sh_vec = sh_mf ? 0 : sh_tiles;
  const int n_tiles = min(tiles_m + tiles_g + sh_tiles, a.max_tiles);
  if (tid < E) {
    const int off = pre_c + c_in - c;
    sm.off[tid] = off;
    sm.it_m[tid] = pre_m + tm_in - tm;
    sm.vt[tid] = (c > 0 && tm == 0) ? mf_tiles + sh_vec + pre_g + tg_in - tg : -1;
    a.counts[tid] = c;
    a.offsets[tid] = off;
  }
  if (tid == 0) {
    sm.off[E] = tot_c;
    a.offsets[E] = tot_c;
  }
  if (tid == 0) {
    // (batches with matrix-core tiles have the standard vector items)
    a.ctl[CTL_N_UP] = n_tiles * vec_up_chunks(T);
    a.ctl[CTL_N_DN] = n_tiles * vec_dn_chunks(T);
    a.ctl[CTL_N_UP_MF] = min(mf_tiles, n_tiles) * mf_up_chunks(bn);
    a.ctl[CTL_N_DN_MF] = min(mf_tiles, n_tiles) * N_DN_CHUNKS;
  }
  __syncthreads();
  // stable permutation and its inverse
  for (int s = tid; s < S; s += nth) {
    const int e = sm.ids[s], t = s / K;
    const uint32_t* me = sm.mask + e * W;
    int r = 0;
    for (int w = 0; w < (t >> 5); ++w) r += __popc(me[w]);
    r += __popc(me[t >> 5] & ((1u << (t & 31)) - 1u));
    const int off = sm.off[e], pos = off + r;
    a.perm[pos] = s;
    a.inv_perm[s] = pos;
    const int v0 = sm.vt[e];
    if (v0 >= 0) {  // vector-path bucket: the token goes into slot r % 4 of tile r / 4
      const int k = r / GV_GROUP, j = r % GV_GROUP, ti = v0 + k;
      if (ti < n_tiles) {
        uint16_t* entry = reinterpret_cast<uint16_t*>(a.tiles + ti);
        entry[4 + j] = (uint16_t)t;
        if (j == 0) {
          uint32_t* w2 = reinterpret_cast<uint32_t*>(a.tiles + ti);
          w2[0] = item_head(e, 0, min(GV_GROUP, sm.off[e + 1] - off - k * GV_GROUP), false);
          w2[1] = (uint32_t)pos;
        }
      }
    }
  }
  // routed matrix-core tiles, one expert per thread (at most T / bn each)
  if (tid < E && tm > 0) {
    const int e = tid, off = sm.off[e];
    for (int k = 0; k < tm; ++k) {
      const int ti = sm.it_m[e] + k;
      if (ti >= n_tiles) break;
      Item it;
      it.head = item_head(e, 0, min(bn, c - k * bn), true);
      it.p0 = (uint32_t)(off + k * bn);
      it.t01 = it.t23 = 0u;
      a.tiles[ti] = it;
    }
  }
  // the shared expert's tiles, on the threads past the experts (a 256-thread
  // caller writes them itself: they do not depend on the routing)
  for (int i = tid - 256; i >= 0 && i < sh_tiles; i += nth - 256) {
    const int ti = (sh_mf ? tiles_m : mf_tiles) + i;
    if (ti >= n_tiles) break;
    a.tiles[ti] = shared_tile(T, i, sh_mf, bn);
  }
}

template <bool TOPK>
__global__ __launch_bounds__(RS_THREADS) void route_small_kernel(LayerArgs a) {
  __shared__ RouteSmallSmem sm;
  static_assert(RS_THREADS > 256 && MAX_E <= 256, "experts on the first four waves, shared tiles on the rest");
  route_small<TOPK>(a, sm);
}

// top-k (with the buckets too, for up to RS_FUSED_T tokens)
hipError_t launch_topk(const LayerArgs& a, hipStream_t s) {
  if (a.T <= RS_FUSED_T) hipLaunchKernelGGL(route_small_kernel<true>, dim3(1), dim3(RS_THREADS), 0, s, a);
  else if (router_splits(a.T) == ROUTER_KS)
    hipLaunchKernelGGL(topk_kernel<ROUTER_KS>, dim3(ceil_div(a.T, TK_THREADS / 64)), dim3(TK_THREADS), 0, s, a);
  else hipLaunchKernelGGL(topk_kernel<ROUTER_KS_L>, dim3(ceil_div(a.T, TK_THREADS / 64)), dim3(TK_THREADS), 0, s, a);
  return hipGetLastError();
}

// buckets and work lists (done by the top-k launch for up to RS_FUSED_T tokens)
hipError_t launch_bucket(const LayerArgs& a, hipStream_t s) {
  if (a.T <= RS_FUSED_T) return hipSuccess;
  if (a.T <= RS_MAX_T) {
    hipLaunchKernelGGL(route_small_kernel<false>, dim3(1), dim3(RS_THREADS), 0, s, a);
    return hipGetLastError();
  }
  const int nch = ceil_div(a.T, BK_CT);
  hipLaunchKernelGGL(chunk_hist_kernel, dim3(nch), dim3(BK_THREADS), 0, s, a);
  hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(BK_THREADS), 0, s, a);
  hipLaunchKernelGGL(chunk_perm_kernel, dim3(nch), dim3(BK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
