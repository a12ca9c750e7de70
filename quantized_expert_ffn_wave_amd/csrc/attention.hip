// Decode attention for the layout of the review "Recursive Flint 40B-A2.5B"
// (orcarouter.ai), section "The architecture is an argument about memory
// bandwidth": 32 query heads share 4 key-value heads of dimension 128 (query
// head h reads key-value head h / 8); sliding-window layers attend to the
// current token and the 512 before it, the others to every earlier token;
// rotary embedding on the sliding-window layers only; an RMSNorm over each head
// of q and k; a learned sink per query head.
//
// One new token per sequence, two kernels on the caller's stream:
//   decode   per (sequence, key-value head, split of positions): RMSNorm (and
//            rotation) of the group's 8 query heads straight into MFMA operands;
//            the wave whose step holds the new position also normalises
//            (rotates) the new key and appends it and the value to the cache;
//            then the 8 query heads against the split's keys and values on the
//            16x16x32 bf16 MFMA, an online softmax, unnormalised partial outputs;
//   combine  per (sequence, query head): the splits and the sink merged (with
//            one split the decode kernel writes the output itself).
//
// Cache layout (bf16), per (sequence, key-value head), in the order the MFMA
// operands read it, so that each quarter-wave's 16-byte loads are contiguous:
//   keys   [cap/16][D/8][16][8]: position p, dimension d at
//          ((p / 16) * 16 + d / 8) * 128 + (p % 16) * 8 + d % 8;
//   values [cap/32][D/16][4][16][8]: position p = 32 a + 16 h + 4 g + s,
//          dimension d at (a * 8 + d / 16) * 512 + g * 128 + (d % 16) * 8 + 4 h + s.
// Both products contract over 16-byte runs (q.k over 8 dimensions of one
// position, p.v over the 8 positions {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3} of
// a 32-position block, the positions whose scores one lane holds), and every
// load instruction of a wave reads 1 KB in one piece.
#include "common.hpp"
#include "attention.hpp"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int AD = ATTN_D;            // head dimension
constexpr int AGQ = ATTN_HQ / ATTN_HK;  // query heads per key-value head (8)
constexpr int ATILE = 64;             // alignment of the attended span's start (positions)
constexpr int ADW = 4;                // waves per decode workgroup
constexpr int ASTEP = 32;             // positions per step of a decode wave
constexpr float LOG2E = 1.4426950408889634f;

__device__ inline u32x4 ld16g(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// the cache is streamed once per step: nontemporal loads keep it from displacing
// other lines in L2 and the last-level cache
__device__ inline u32x4 ld16nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }

// element offsets within one (sequence, key-value head) block of the caches
__device__ inline size_t k_off(int p, int d) { return ((size_t)(p >> 4) * 16 + (d >> 3)) * 128 + (p & 15) * 8 + (d & 7); }
__device__ inline size_t v_off(int p, int d) {
  return ((size_t)(p >> 5) * 8 + (d >> 4)) * 512 + ((p >> 2) & 3) * 128 + (d & 15) * 8 + ((p >> 4) & 1) * 4 + (p & 3);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// ---- decode ------------------------------------------------------------------------
// One workgroup of 4 waves per (split, key-value head, sequence).  The attended
// positions are cut into steps of 32 from the window's start rounded down to 64;
// step q goes to split (q / 4) mod splits and wave q mod 4, so that the waves of
// all splits stream adjacent steps together.  A wave keeps the next step's 16
// loads in flight while it multiplies the current one, and the waves' running
// maxima, sums and outputs are merged through LDS at the end.
// Lane (c, g) = (lane % 16, lane / 16).  Step of 32 positions t0 ..:
//   scores on 2 MFMA tiles (t < 2) x 4 K-steps: A = keys, row r of tile t is
//   position t0 + 16 t + r, lane (r, g) supplying d = 32 i + 8 g .. + 7 of K-step
//   i; B = q of head c (zero for c >= 8), the same d.  Output lane (c, g) holds
//   the scores of head c at positions t0 + 16 t + 4 g + j, j < 4;
//   values on 8 MFMA tiles of 16 dimensions: A = V^T, lane (r, g) supplying
//   dimension 16 dt + r at those 8 positions (16 contiguous bytes); B = the
//   lane's own 8 probabilities of head c.  Output
//   lane (c, g) holds O[head c][16 dt + 4 g + j].
// cos and sin of the rotation angle pos * inv_freq: the angle in revolutions is
// formed and reduced to [-1/2, 1/2] in fp64 (positions reach 10^5, where an fp32
// angle would be off by 10^-2 rad), then v_cos_f32 / v_sin_f32 take it in
// revolutions (absolute error near 1e-6, against a bf16 step of 4e-3).
__device__ inline void rotation(double inv_freq, int pos, float& cs, float& sn) {
  const double rev = (double)pos * inv_freq * 0.15915494309189535;  // 1 / (2 pi)
  const float fr = (float)(rev - rint(rev));
  cs = __builtin_amdgcn_cosf(fr);
  sn = __builtin_amdgcn_sinf(fr);
}

// The prepared head (query or key) in the decode's operand layout: lane (c, g)
// holds d = 32 i + 8 g + e (i < 4, e < 8).  The 4 lanes of a head (g = 0 .. 3)
// together hold its 128 elements, and element d and its rotation partner
// d + 64 (i and i + 2) sit in the same lane.  Split in two so that the inputs'
// loads can go out ahead of the cache's: loads, then the norm and rotation.
struct QIn {
  u32x4 x[4], gain[4];
};

// src: the head's 128 bf16 elements, or null for a lane that holds no head
__device__ inline void prep_load(const uint16_t* src, const uint16_t* gain, int g, QIn& in) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    in.x[i] = src ? ld16g(src + 8 * g + 32 * i) : u32x4{0u, 0u, 0u, 0u};
    in.gain[i] = ld16g(gain + 8 * g + 32 * i);
  }
}

// The rotation frequency theta^(-d/64) of element d = 32 i + 8 g + e, as the
// product of theta^(-e/64), theta^(-8g/64) and theta^(-32i/64) formed in fp64 on
// the host (two fp64 roundings: a relative error near 2^-52)
__device__ inline double freq(const AttnArgs& a, int i, int e, double fg) {
  return (i ? a.rot_32 : 1.0) * a.rot_e[e] * fg;
}

__device__ inline void prep(const AttnArgs& a, const QIn& in, bool live, int g, int pos, u32x4 (&out)[4]) {
  float y[4][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[i][e] = bf16_to_f32((uint16_t)(in.x[i][e >> 1] >> (16 * (e & 1))));
      ss += y[i][e] * y[i][e];
    }
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  const float r = live ? rsqrtf(ss * (1.f / AD) + a.eps) : 0.f;  // lanes without a head stay 0, even with eps = 0
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) y[i][e] *= r * bf16_to_f32((uint16_t)(in.gain[i][e >> 1] >> (16 * (e & 1))));
  if (a.rope) {
    const double fg = g == 0 ? a.rot_g[0] : g == 1 ? a.rot_g[1] : g == 2 ? a.rot_g[2] : a.rot_g[3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float cs, sn;
        rotation(freq(a, i, e, fg), pos, cs, sn);
        const float t0 = y[i][e] * cs - y[i + 2][e] * sn, t1 = y[i + 2][e] * cs + y[i][e] * sn;
        y[i][e] = t0;
        y[i + 2][e] = t1;
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      out[i][e] = (uint32_t)f32_to_bf16(y[i][2 * e]) | ((uint32_t)f32_to_bf16(y[i][2 * e + 1]) << 16);
}

struct AStep {
  u32x4 k[2][4];
  u32x4 v[AD / 16];
};

__global__ __launch_bounds__(64 * ADW, 2) void attn_decode_kernel(AttnArgs a) {
  __shared__ float sm_ml[ADW][2][16];
  __shared__ f32x4 sm_o[ADW - 1][AD / 16][64];
  const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int len = min(max(a.pos[b], 0), a.cap - 1) + 1;
  const int lo = (a.window > 0 && len > a.window) ? len - a.window : 0;
  const int base = lo & ~(ATILE - 1);
  // steps of 32 positions from base; step q belongs to split (q / ADW) % splits
  // and wave q % ADW, so that the splits' waves read adjacent steps at once
  const int nst = (len - base + ASTEP - 1) / ASTEP;
  const int first_step = split * ADW + wave, stride = a.splits * ADW;
  const int nsteps = first_step < nst ? (nst - first_step + stride - 1) / stride : 0;
  const int hq = kv * AGQ + c;
  const int pos = len - 1;
  // the new token's key and value: appended by the one wave whose step holds
  // its position, before that wave's cache loads (a fence orders its stores
  // before its loads; no other wave reads these cache lines: a 32-position step
  // belongs to one wave, and its lines hold that step's positions only)
  const int pos_step = (pos - base) / ASTEP;
  if ((pos_step / ADW) % a.splits == split && pos_step % ADW == wave) {
    // lanes (0, g) prepare the key; its 8-element runs are contiguous in the key cache
    QIn kin;
    prep_load(c == 0 ? a.k + ((size_t)b * ATTN_HK + kv) * AD : nullptr, a.k_gain, g, kin);
    const uint16_t* vs = a.v + ((size_t)b * ATTN_HK + kv) * AD;
    u32x4 vv[4];  // the value's same 32 elements, loaded with the key's inputs
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = (c == 0) ? ld16g(vs + 32 * i + 8 * g) : u32x4{0u, 0u, 0u, 0u};
    u32x4 kp[4];
    prep(a, kin, c == 0, g, pos, kp);
    if (c == 0) {
      uint16_t* kd = a.k_cache + ((size_t)b * ATTN_HK + kv) * (size_t)a.cap * AD;
      uint16_t* vd = a.v_cache + ((size_t)b * ATTN_HK + kv) * (size_t)a.cap * AD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(kd + k_off(pos, 32 * i + 8 * g)) = kp[i];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vd[v_off(pos, 32 * i + 8 * g + e)] = (uint16_t)(vv[i][e >> 1] >> (16 * (e & 1)));
      }
    }
    __threadfence_block();  // the stores complete before this wave's loads
  }
  const uint16_t* kbase = a.k_cache + ((size_t)b * ATTN_HK + kv) * (size_t)a.cap * AD;
  const uint16_t* vbase = a.v_cache + ((size_t)b * ATTN_HK + kv) * (size_t)AD * a.cap;
  // start of the wave's step j, clamped to its last step: with an odd step
  // count the second buffer of the last pair reloads that step (never used),
  // so that every load is issued and the waits stay exact
  auto step_pos = [&](int j) { return base + ASTEP * (first_step + stride * min(j, nsteps - 1)); };
  auto load = [&](AStep& st, int t0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int p = t0 + 16 * t + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.k[t][i] = ld16nt(kbase + k_off(p, 32 * i + 8 * g));
    }
#pragma unroll
    for (int dt = 0; dt < AD / 16; ++dt) st.v[dt] = ld16nt(vbase + v_off(t0 + 4 * g, 16 * dt + c));
  };
  // the query's inputs, then the first two steps, are loaded before the query
  // is prepared, so that its norm and rotation overlap the cache loads
  QIn qin;
  prep_load(c < AGQ ? a.q + ((size_t)b * ATTN_HQ + hq) * AD : nullptr, a.q_gain, g, qin);
  AStep s0, s1;
  if (nsteps > 0) {
    load(s0, step_pos(0));
    load(s1, step_pos(1));
  }
  u32x4 qv[4];  // this lane's prepared query operand: head c, d = 32 i + 8 g .. + 7
  prep(a, qin, c < AGQ, g, pos, qv);
  if (split == 0 && c < AGQ && wave == 0) {  // q' also to the workspace, for inspection
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(a.qbuf + ((size_t)b * ATTN_HQ + hq) * AD + 8 * g + 32 * i) = qv[i];
  }
  float m = -INFINITY, l = 0.f;
  f32x4 o[AD / 16];
#pragma unroll
  for (int dt = 0; dt < AD / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (nsteps > 0) {
    const float qscale = LOG2E * rsqrtf((float)AD);  // scores in the log2 domain
    auto compute = [&](const AStep& st, int t0, bool valid) {
      // scores of positions t0 + 8 g + e, masked outside [lo, len); an invalid
      // step (past the wave's last, loaded again only to keep the waits exact)
      // is masked whole
      const int lo_v = valid ? lo : len;
      float sc[8];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st.k[t][i]),
                                                        __builtin_bit_cast(bf16x8, qv[i]), acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = t0 + 16 * t + 4 * g + j;
          sc[4 * t + j] = (p >= lo_v && p < len) ? acc[j] * qscale : -INFINITY;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      // a step wholly before the window's start leaves the maximum at -inf
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < AD / 16; ++dt) o[dt] *= alpha;
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        // the denominator sums the same bf16 probabilities the products use
        const uint16_t p0 = f32_to_bf16(exp2f(sc[e] - m_use)), p1 = f32_to_bf16(exp2f(sc[e + 1] - m_use));
        l += bf16_to_f32(p0) + bf16_to_f32(p1);
        pk[e / 2] = (uint32_t)p0 | ((uint32_t)p1 << 16);
      }
      // positions outside [lo, len) carry probability 0; their values are zeroed
      // too, so that whatever the unwritten cache holds cannot turn into NaN
      const int pv0 = t0 + 4 * g;  // element e of the lane's 8 is position pv0 + 16 (e / 4) + e % 4
      const bool whole = pv0 >= lo_v && pv0 + 20 <= len;
      const u32x4 pb = u32x4{pk[0], pk[1], pk[2], pk[3]};
#pragma unroll
      for (int dt = 0; dt < AD / 16; ++dt) {
        u32x4 v = st.v[dt];
        if (!whole) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int p = pv0 + 16 * (e >> 1) + 2 * (e & 1);  // elements 2 e, 2 e + 1
            const uint32_t keep =
                ((p >= lo_v && p < len) ? 0x0000FFFFu : 0u) | ((p + 1 >= lo_v && p + 1 < len) ? 0xFFFF0000u : 0u);
            v[e] &= keep;
          }
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), __builtin_bit_cast(bf16x8, pb),
                                                        o[dt], 0, 0, 0);
      }
    };
    // two steps in flight: the same loads outstanding at the loop's entry, at
    // its back edge and after it, so each compute waits only for its own
    // step's loads; the last pair (or single step) is computed after the loop
    // and issues no loads
    int j = 0;
    for (; j + 2 < nsteps; j += 2) {
      compute(s0, step_pos(j), true);
      load(s0, step_pos(j + 2));
      compute(s1, step_pos(j + 1), true);
      load(s1, step_pos(j + 3));
    }
    compute(s0, step_pos(j), true);
    if (j + 1 < nsteps) compute(s1, step_pos(j + 1), true);
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
      sc[w] = (M == -INFINITY || sm_ml[w][0][c] == -INFINITY) ? 0.f : exp2f(sm_ml[w][0][c] - M);
      L += sc[w] * sm_ml[w][1][c];
    }
    if (a.splits == 1) {
      // one split: the workgroup holds every attended position, so it adds the
      // sink and writes the output itself (the launcher skips the combine)
      const float z = a.sinks ? a.sinks[hq] * LOG2E : -INFINITY;
      const float M2 = fmaxf(M, z);
      const float wm = exp2f(M - M2);
      const float inv = 1.f / (L * wm + (a.sinks ? exp2f(z - M2) : 0.f));
      uint16_t* po = a.out + ((size_t)b * ATTN_HQ + hq) * AD;
#pragma unroll
      for (int dt = 0; dt < AD / 16; ++dt) {
        f32x4 acc = o[dt] * sc[0];
#pragma unroll
        for (int w = 1; w < ADW; ++w) acc += sm_o[w - 1][dt][lane] * sc[w];
        const float f = wm * inv;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(acc[0] * f) | ((uint32_t)f32_to_bf16(acc[1] * f) << 16);
        pk.y = (uint32_t)f32_to_bf16(acc[2] * f) | ((uint32_t)f32_to_bf16(acc[3] * f) << 16);
        *reinterpret_cast<uint2*>(po + 16 * dt + 4 * g) = pk;
      }
    } else {
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
  hipLaunchKernelGGL(attn_decode_kernel, dim3(a.splits, ATTN_HK, B), dim3(64 * ADW), 0, s, a);
  if (a.splits > 1) hipLaunchKernelGGL(attn_combine_kernel, dim3(B * ATTN_HQ), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
