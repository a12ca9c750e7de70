// Decode attention for the layout of the review "Recursive Flint 40B-A2.5B"
// (orcarouter.ai), section "The architecture is an argument about memory
// bandwidth": 32 query heads share 4 key-value heads of dimension 128 (query
// head h reads key-value head h / 8); sliding-window layers attend to the
// current token and the 512 before it, the others to every earlier token;
// rotary embedding on the sliding-window layers only; an RMSNorm over each head
// of q and k; a learned sink per query head.
//
// One new token per sequence, three kernels on the caller's stream:
//   prep     per sequence: RMSNorm (and rotation) of the token's 32 q and 4 k
//            heads, q' to the workspace, k' and v appended to the cache at the
//            token's position;
//   decode   per (sequence, key-value head, split of positions): the 8 query
//            heads of the group against the split's keys and values on the
//            16x16x32 bf16 MFMA, an online softmax, unnormalised partial outputs;
//   combine  per (sequence, query head): the splits and the sink merged.
//
// Cache layout (bf16): keys [B][HK][cap][D] (a position's 128 elements
// contiguous), values transposed in tiles of 64 positions [B][HK][cap/64][D][64]
// (within a tile, a dimension's positions contiguous, and the tile's 16 KB in
// one piece), so that both products contract over contiguous memory: q.k over
// d, p.v over positions.
#include "common.hpp"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int AD = ATTN_D;            // head dimension
constexpr int AGQ = ATTN_HQ / ATTN_HK;  // query heads per key-value head (8)
constexpr int ATILE = 64;             // positions per tile of the decode loop
constexpr int ADW = 4;                // waves per decode workgroup (a tile each, in turn)
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline u32x4 ld16g(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// ---- prep --------------------------------------------------------------------------
// One wave per head (grid B x 9 workgroups of 4 waves: 32 q heads, then 4 k
// heads), lane l holding elements l and l + 64 (the rotation's pair), so that
// every head's load, norm and store run side by side.  The rotation angle
// pos * inv_freq[l] (inv_freq formed in fp64 on the host) is reduced modulo 2 pi
// in fp64: positions reach 10^5, where an fp32 angle would be off by 10^-2 rad.
__global__ __launch_bounds__(256) void attn_prep_kernel(AttnArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int pos = min(max(a.pos[b], 0), a.cap - 1);
  const bool isq = h < ATTN_HQ;
  const uint16_t* src = isq ? a.q + ((size_t)b * ATTN_HQ + h) * AD : a.k + ((size_t)b * ATTN_HK + (h - ATTN_HQ)) * AD;
  const uint16_t* gain = isq ? a.q_gain : a.k_gain;
  const float x0 = bf16_to_f32(src[lane]), x1 = bf16_to_f32(src[lane + 64]);
  const float g0 = bf16_to_f32(gain[lane]), g1 = bf16_to_f32(gain[lane + 64]);
  const float r = rsqrtf(wave_sum(x0 * x0 + x1 * x1) * (1.f / AD) + a.eps);
  float y0 = x0 * r * g0, y1 = x1 * r * g1;
  if (a.rope) {
    const double two_pi = 6.283185307179586;
    const double ang = (double)pos * a.inv_freq[lane];
    const float red = (float)fma(-rint(ang * (1.0 / two_pi)), two_pi, ang);  // in [-pi, pi]
    float sn, cs;
    sincosf(red, &sn, &cs);
    const float t0 = y0 * cs - y1 * sn, t1 = y1 * cs + y0 * sn;
    y0 = t0;
    y1 = t1;
  }
  uint16_t* dst = isq ? a.qbuf + ((size_t)b * ATTN_HQ + h) * AD
                      : a.k_cache + (((size_t)b * ATTN_HK + (h - ATTN_HQ)) * a.cap + pos) * AD;
  dst[lane] = f32_to_bf16(y0);
  dst[lane + 64] = f32_to_bf16(y1);
  if (blockIdx.y == 0) {  // values as given, one element per (head, dimension), into the transposed tiles
    for (int i = threadIdx.x; i < ATTN_HK * AD; i += 256) {
      const int kv = i / AD, d = i % AD;
      a.v_cache[(((size_t)b * ATTN_HK + kv) * (a.cap / ATILE) + pos / ATILE) * (AD * ATILE) + d * ATILE + pos % ATILE] =
          a.v[((size_t)b * ATTN_HK + kv) * AD + d];
    }
  }
}

// ---- decode ------------------------------------------------------------------------
// One workgroup of 4 waves per (split, key-value head, sequence); wave w takes
// the split's tiles w, w + 4, .. and the waves' running maxima, sums and outputs
// are merged through LDS at the end.  Lane (c, g) = (lane % 16, lane / 16).
// Tile of 64 positions t0 ..:
//   scores on 4 MFMA tiles (t < 4) x 4 K-steps: A = keys, row r of tile t is
//   position t0 + 32 (t / 2) + 8 (r / 4) + 4 (t % 2) + r % 4, lane (r, g)
//   supplying d = 8 g + 32 i .. + 7 of step i; B = q of head c (zero for c >= 8),
//   the same d.  Output lane (c, g) holds the scores of head c at positions
//   t0 + 32 (t / 2) + 8 g + 4 (t % 2) + j, j < 4: for each 32-position half
//   the 8 positions t0 + 32 h + 8 g .. + 7;
//   values on 2 halves x 8 MFMA tiles of 16 dimensions: A = V^T, lane (r, g)
//   supplying dimension 16 dt + r at the positions of its k-group, 8 g .. + 7 of
//   the half (16 contiguous bytes of the tile); B = the lane's own 8
//   probabilities of head c.  Output lane (c, g) holds O[head c][16 dt + 4 g + j].
__global__ __launch_bounds__(64 * ADW) void attn_decode_kernel(AttnArgs a) {
  __shared__ float sm_ml[ADW][2][16];
  __shared__ f32x4 sm_o[ADW - 1][AD / 16][64];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int len = min(max(a.pos[b], 0), a.cap - 1) + 1;
  const int lo = (a.window > 0 && len > a.window) ? len - a.window : 0;
  const int base = lo & ~(ATILE - 1);
  const int p_begin = base + split * a.chunk, p_end = min(len, p_begin + a.chunk);
  const int hq = kv * AGQ + c;
  float m = -INFINITY, l = 0.f;
  f32x4 o[AD / 16];
#pragma unroll
  for (int dt = 0; dt < AD / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p_begin + wave * ATILE < p_end) {
    u32x4 qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      qv[i] = (c < AGQ) ? ld16g(a.qbuf + ((size_t)b * ATTN_HQ + hq) * AD + 8 * g + 32 * i) : u32x4{0u, 0u, 0u, 0u};
    const uint16_t* kbase = a.k_cache + ((size_t)b * ATTN_HK + kv) * (size_t)a.cap * AD;
    const uint16_t* vbase = a.v_cache + ((size_t)b * ATTN_HK + kv) * (size_t)AD * a.cap;  // this head's tiles
    const float qscale = LOG2E * rsqrtf((float)AD);  // scores in the log2 domain
    for (int t0 = p_begin + wave * ATILE; t0 < p_end; t0 += ADW * ATILE) {
      // all loads of the tile first
      u32x4 kv4[4][4], vt[2][AD / 16];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int p = t0 + 32 * (t >> 1) + 8 * (c >> 2) + 4 * (t & 1) + (c & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) kv4[t][i] = ld16g(kbase + (size_t)p * AD + 8 * g + 32 * i);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int dt = 0; dt < AD / 16; ++dt)
          vt[h][dt] = ld16g(vbase + (size_t)t0 * AD + (16 * dt + c) * ATILE + 32 * h + 8 * g);
      // scores, masked outside [lo, len)
      float sc[2][8];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv4[t][i]),
                                                        __builtin_bit_cast(bf16x8, qv[i]), acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = t0 + 32 * (t >> 1) + 8 * g + 4 * (t & 1) + j;
          sc[t >> 1][4 * (t & 1) + j] = (p >= lo && p < len) ? acc[j] * qscale : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sc[h][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);  // finite: every tile holds at least one position in range
      const float alpha = exp2f(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < AD / 16; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // the denominator sums the same bf16 probabilities the products use
          const uint16_t p0 = f32_to_bf16(exp2f(sc[h][e] - m_new)), p1 = f32_to_bf16(exp2f(sc[h][e + 1] - m_new));
          l += bf16_to_f32(p0) + bf16_to_f32(p1);
          pk[e / 2] = (uint32_t)p0 | ((uint32_t)p1 << 16);
        }
        // positions outside [lo, len) carry probability 0; their values are zeroed
        // too, so that whatever the unwritten cache holds cannot turn into NaN
        const int pv0 = t0 + 32 * h + 8 * g;
        const bool whole = pv0 >= lo && pv0 + 8 <= len;
        const u32x4 pb = u32x4{pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
        for (int dt = 0; dt < AD / 16; ++dt) {
          u32x4 v = vt[h][dt];
          if (!whole) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int p = pv0 + 2 * e;
              const uint32_t keep = ((p >= lo && p < len) ? 0x0000FFFFu : 0u) | ((p + 1 >= lo && p + 1 < len) ? 0xFFFF0000u : 0u);
              v[e] &= keep;
            }
          }
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), __builtin_bit_cast(bf16x8, pb),
                                                          o[dt], 0, 0, 0);
        }
      }
    }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
  }
  // merge the waves' running states: M = max m_w, each scaled by 2^(m_w - M)
  if (g == 0) {
    sm_ml[wave][0][c] = m;
    sm_ml[wave][1][c] = l;
  }
  if (wave > 0) {
#pragma unroll
    for (int dt = 0; dt < AD / 16; ++dt) sm_o[wave - 1][dt][lane] = o[dt];
  }
  __syncthreads();
  if (wave == 0 && c < AGQ) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < ADW; ++w) M = fmaxf(M, sm_ml[w][0][c]);
    float L = 0.f;
    float sc[ADW];
#pragma unroll
    for (int w = 0; w < ADW; ++w) {
      // waves without positions hold m = -inf, l = 0, o = 0
      sc[w] = (M == -INFINITY) ? 0.f : exp2f(sm_ml[w][0][c] - M);
      L += sc[w] * sm_ml[w][1][c];
    }
    const size_t row = ((size_t)b * ATTN_HQ + hq) * a.splits + split;
    float* po = a.part_o + row * AD;
#pragma unroll
    for (int dt = 0; dt < AD / 16; ++dt) {
      f32x4 acc = o[dt] * sc[0];
#pragma unroll
      for (int w = 1; w < ADW; ++w) acc += sm_o[w - 1][dt][lane] * sc[w];
      *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = acc;
    }
    if (g == 0) {
      a.part_ml[2 * row] = M;
      a.part_ml[2 * row + 1] = L;
    }
  }
}

// ---- combine -----------------------------------------------------------------------
// One wave per (sequence, query head); lane l owns dimensions 2 l, 2 l + 1.
// out = sum_s 2^(m_s - M) o_s / (sum_s 2^(m_s - M) l_s + 2^(z log2 e - M)).
// There are at most 64 splits (the plan's chunk grows to keep it so): lane s
// reads split s's maximum and sum, and the splits' outputs are loaded 32 at a
// time with their weights read from the owning lanes.
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int bh = blockIdx.x, lane = threadIdx.x, S = a.splits;
  const float* ml = a.part_ml + (size_t)bh * S * 2;
  const float z = a.sinks ? a.sinks[bh % ATTN_HQ] * LOG2E : -INFINITY;
  const float ms = lane < S ? ml[2 * lane] : -INFINITY, ls = lane < S ? ml[2 * lane + 1] : 0.f;
  float M = fmaxf(ms, z);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));
  const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);  // splits past the end hold -inf
  const float den = wave_sum(w * ls) + (a.sinks ? exp2f(z - M) : 0.f);
  const float* po = a.part_o + (size_t)bh * S * AD + 2 * lane;
  float o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < S; s0 += 32) {
    float2 v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i)
      v[i] = (s0 + i < S) ? *reinterpret_cast<const float2*>(po + (size_t)(s0 + i) * AD) : make_float2(0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s0 + i));
      o0 += wi * v[i].x;
      o1 += wi * v[i].y;
    }
  }
  const float inv = 1.f / den;
  a.out[(size_t)bh * AD + 2 * lane] = f32_to_bf16(o0 * inv);
  a.out[(size_t)bh * AD + 2 * lane + 1] = f32_to_bf16(o1 * inv);
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL(attn_prep_kernel, dim3(B, (ATTN_HQ + ATTN_HK) / 4), dim3(256), 0, s, a);
  hipLaunchKernelGGL(attn_decode_kernel, dim3(a.splits, ATTN_HK, B), dim3(64 * ADW), 0, s, a);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(B * ATTN_HQ), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
