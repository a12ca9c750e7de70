// Expert FFN: gate/up projection with fused SwiGLU, and down projection, over
// the expert buckets.  Both kernels are persistent: each workgroup walks the
// device-side work list written by the bucket kernel.  Items of small buckets
// (<= GEMV_MAX tokens) run on the vector ALUs, streaming packed weight rows
// with 16-byte loads and decoding them in registers; items of large buckets
// run on the matrix cores, decoding a weight tile into LDS once and
// multiplying it with every token tile.
//
// The review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", argues that decoding
// this model is a weight-movement problem; the small-bucket path is therefore
// built to move each touched weight byte from HBM exactly once, with the
// arithmetic kept under the HBM time.  Expert form (SwiGLU, width 512) and
// the 4-bit layouts are the readings documented in include/moe_ffn.h.
#include "common.hpp"

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte load of weight bytes that are read once (non-temporal hint).
__device__ inline u32x4 ld_stream(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// E2M1 pair (byte B of w) -> fp16 pair, unscaled.
template <int B> __device__ inline uint32_t fp4x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

constexpr uint32_t MAGIC = 0x64006400u;  // fp16 pair (1024, 1024): ORing a nibble into the
                                         // low mantissa bits gives 1024 + q exactly

__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ inline float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_f16x2(a), as_f16x2(b), c, false);
}
__device__ inline float dot2b(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// two bf16 (lo, hi halves of v) -> packed fp16 pair (exact for normal-range values)
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u)));
}

// natural pairs N0=(e0,e1) N1=(e2,e3) N2=(e4,e5) N3=(e6,e7) -> the order the
// q4_1 nibble split produces: (e0,e4) (e1,e5) (e2,e6) (e3,e7)
__device__ inline void q4_order(uint32_t n0, uint32_t n1, uint32_t n2, uint32_t n3, uint32_t* o) {
  o[0] = __builtin_amdgcn_perm(n2, n0, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(n2, n0, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(n3, n1, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(n3, n1, 0x07060302u);
}

__device__ inline float f16lo(uint32_t v) { return (float)as_f16x2(v)[0]; }
__device__ inline float f16hi(uint32_t v) { return (float)as_f16x2(v)[1]; }

// Saturating fp32 -> fp16 pair (the SwiGLU output is stored as fp16).
__device__ inline uint32_t pack_h16(float a, float b) {
  a = fminf(fmaxf(a, -65504.f), 65504.f);
  b = fminf(fmaxf(b, -65504.f), 65504.f);
  f16x2 r = {(_Float16)a, (_Float16)b};
  return as_u32(r);
}
__device__ inline uint32_t pack_b16(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// ======================================================================================
// Format traits for the vector (GEMV) path.  Each lane owns one 32-element chunk
// of a row: 16 bytes of 4-bit codes (or 64 bytes of bf16).
// ======================================================================================
template <int FMT> struct GV;

template <> struct GV<FMT_Q4_1> {
  // raw chunk: 16 B codes + {d, m}
  struct Raw { u32x4 c; uint32_t dm; };
  // activations for one chunk: fp16 pairs in nibble order + even/odd sums
  struct X { uint32_t p[16]; float se, so; };
  static __device__ Raw load(const QMat& q, size_t row, int chunk, int cols) {
    Raw r;
    r.c = ld_stream(q.codes + row * (cols / 2) + 16 * chunk);
    r.dm = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(q.scales) + row * (cols / 32) + chunk);
    return r;
  }
  // src: 16 dwords of fp16 pairs, natural order
  static __device__ void prep(X& x, const uint32_t* src) {
    float se = 0.f, so = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q4_order(src[4 * j], src[4 * j + 1], src[4 * j + 2], src[4 * j + 3], &x.p[4 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) { se += f16lo(src[4 * j + i]); so += f16hi(src[4 * j + i]); }
    }
    x.se = se;
    x.so = so;
  }
  struct U { uint32_t A[4], B[4], C[4], D[4]; float c1, c2, c3, c4; };
  static __device__ void unpack(U& u, const Raw& r, float /*ts*/) {
    const uint32_t w[4] = {r.c[0], r.c[1], r.c[2], r.c[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w8 = w[j] >> 8;
      u.A[j] = (w[j] & 0x000F000Fu) | MAGIC;   // (1024+q0, 1024+q4)
      u.B[j] = (w[j] & 0x00F000F0u) | MAGIC;   // (1024+16q1, 1024+16q5)
      u.C[j] = (w8 & 0x000F000Fu) | MAGIC;     // (1024+q2, 1024+q6)
      u.D[j] = (w8 & 0x00F000F0u) | MAGIC;     // (1024+16q3, 1024+16q7)
    }
    const float d = f16lo(r.dm), m = f16hi(r.dm);
    // block dot = d*lo + (d/16)*hi + (m - 1024 d)*sum_even + (m - 64 d)*sum_odd
    u.c1 = d;
    u.c2 = d * 0.0625f;
    u.c3 = m - 1024.f * d;
    u.c4 = m - 64.f * d;
  }
  static __device__ float dot(const U& u, const X& x) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo = dot2h(u.A[j], x.p[4 * j + 0], lo);
      hi = dot2h(u.B[j], x.p[4 * j + 1], hi);
      lo = dot2h(u.C[j], x.p[4 * j + 2], lo);
      hi = dot2h(u.D[j], x.p[4 * j + 3], hi);
    }
    return u.c1 * lo + u.c2 * hi + u.c3 * x.se + u.c4 * x.so;
  }
};

template <> struct GV<FMT_NVFP4> {
  struct Raw { u32x4 c; uint32_t s; };
  struct X { uint32_t p[16]; };
  static __device__ Raw load(const QMat& q, size_t row, int chunk, int cols) {
    Raw r;
    r.c = ld_stream(q.codes + row * (cols / 2) + 16 * chunk);
    r.s = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(q.scales) +
                                                                        row * (cols / 16)) + chunk);
    return r;
  }
  static __device__ void prep(X& x, const uint32_t* src) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x.p[i] = src[i];
  }
  struct U { uint32_t P[16]; float s0, s1; };
  static __device__ void unpack(U& u, const Raw& r, float ts) {
    const uint32_t w[4] = {r.c[0], r.c[1], r.c[2], r.c[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u.P[4 * j + 0] = fp4x2_to_f16x2<0>(w[j]);
      u.P[4 * j + 1] = fp4x2_to_f16x2<1>(w[j]);
      u.P[4 * j + 2] = fp4x2_to_f16x2<2>(w[j]);
      u.P[4 * j + 3] = fp4x2_to_f16x2<3>(w[j]);
    }
    u.s0 = __builtin_amdgcn_cvt_f32_fp8(r.s, 0) * ts;
    u.s1 = __builtin_amdgcn_cvt_f32_fp8(r.s, 1) * ts;
  }
  static __device__ float dot(const U& u, const X& x) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a0 = dot2h(u.P[i], x.p[i], a0);
#pragma unroll
    for (int i = 8; i < 16; ++i) a1 = dot2h(u.P[i], x.p[i], a1);
    return u.s0 * a0 + u.s1 * a1;
  }
};

template <> struct GV<FMT_BF16> {
  struct Raw { u32x4 c[4]; };
  struct X { uint32_t p[16]; };
  static __device__ Raw load(const QMat& q, size_t row, int chunk, int cols) {
    Raw r;
    const uint8_t* p = q.codes + row * cols * 2 + 64 * chunk;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = ld_stream(p + 16 * i);
    return r;
  }
  static __device__ void prep(X& x, const uint32_t* src) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x.p[i] = src[i];
  }
  struct U { uint32_t P[16]; };
  static __device__ void unpack(U& u, const Raw& r, float) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u.P[4 * i] = r.c[i][0]; u.P[4 * i + 1] = r.c[i][1]; u.P[4 * i + 2] = r.c[i][2]; u.P[4 * i + 3] = r.c[i][3];
    }
  }
  static __device__ float dot(const U& u, const X& x) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = dot2b(u.P[i], x.p[i], a);
    return a;
  }
};

// Operand precision of the expert GEMMs: fp16 for the 4-bit formats (their
// decoded values are exact in fp16), bf16 for bf16 weights.
template <int FMT> constexpr bool OPER_F16 = FMT != FMT_BF16;

// 32 activation elements of one lane as 16 dwords of operand pairs, natural
// order.  src points at bf16 (x) or at the stored SwiGLU output (fp16 for the
// 4-bit formats, bf16 otherwise).
template <int FMT> __device__ inline void load_act(uint32_t* d, const uint16_t* src, bool src_bf16) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = p[i];
    d[4 * i] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
  }
  if (OPER_F16<FMT> && src_bf16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = bf16x2_to_f16x2(d[i]);
  }
}

// Transposing wave reduction: P partials per lane, summed over groups of G
// lanes (xor masks G/2 .. 1).  While more than one value is left, each step
// halves the count: lanes with the mask bit clear keep the first half, lanes
// with it set the second half.  Afterwards v[0] of a lane holds the total of
// index idx(lane) = sum over halving steps s of bit(lane, G>>(s+1)) * P>>(s+1).
template <int P, int G>
__device__ inline void xreduce(float* v) {
  const int lane = threadIdx.x & 63;
  int n = P;
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) {
    if (n > 1) {
      const bool hi = (lane & m) != 0;
      const int h = n / 2;
#pragma unroll
      for (int i = 0; i < P / 2; ++i) {
        if (i < h) {
          const float keep = hi ? v[i + h] : v[i];
          const float send = hi ? v[i] : v[i + h];
          v[i] = keep + __shfl_xor(send, m);
        }
      }
      n = h;
    } else {
      v[0] += __shfl_xor(v[0], m);
    }
  }
}

// Index a lane holds after xreduce<P, G>, and whether it is the lane of its
// group that should write it (the bits of the non-halving steps are zero).
template <int P, int G>
__device__ inline int xreduce_index(int lane, bool& writer) {
  int idx = 0, n = P, plain_mask = 0;
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) {
    if (n > 1) {
      n /= 2;
      if (lane & m) idx += n;
    } else {
      plain_mask |= m;
    }
  }
  writer = (lane & plain_mask) == 0;
  return idx;
}

// Tokens of an item: bucket positions p0 .. p0+cnt-1 of a routed expert (token
// = perm[p] / K, output row p), or tokens t0 .. t0+cnt-1 for the shared expert
// (output row S + t).
struct ItemTok {
  int p0, cnt;
  bool shared;
};

__device__ inline ItemTok item_tokens(const LayerArgs& a, int e, int tile) {
  ItemTok r;
  if (e >= a.E) {
    r.shared = true;
    r.p0 = tile * MFMA_BN;
    r.cnt = a.T - r.p0;
  } else {
    r.shared = false;
    const int c = a.counts[e];
    r.p0 = a.offsets[e] + tile * MFMA_BN;
    r.cnt = c - tile * MFMA_BN;
  }
  if (r.cnt > MFMA_BN) r.cnt = MFMA_BN;
  return r;
}
__device__ inline int tok_of(const LayerArgs& a, const ItemTok& it, int i) {
  return it.shared ? it.p0 + i : a.perm[it.p0 + i] / a.K;
}
__device__ inline int row_of(const LayerArgs& a, const ItemTok& it, int i) {
  return it.shared ? a.S + it.p0 + i : it.p0 + i;
}

// ======================================================================================
// GEMV items
// ======================================================================================

// gate/up + SwiGLU: each wave handles NR row pairs; a lane owns 32-element chunk
// `lane` of the 2048-long rows.
template <int FMT, int M, int NR>
__device__ void gemv_up(const LayerArgs& a, const QMat& G, const QMat& Uq, int mat, const ItemTok& it, int n0) {
  using F = GV<FMT>;
  const int lane = threadIdx.x & 63;
  typename F::X x[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    uint32_t src[16];
    if (t < it.cnt) {
      const int tok = tok_of(a, it, t);
      load_act<FMT>(src, a.x + (size_t)tok * D_MODEL + 32 * lane, true);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) src[i] = 0u;
    }
    F::prep(x[t], src);
  }
  const float tsg = (FMT == FMT_NVFP4) ? G.ts[mat] : 1.f;
  const float tsu = (FMT == FMT_NVFP4) ? Uq.ts[mat] : 1.f;
  typename F::Raw rg[NR], ru[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const size_t row = (size_t)mat * D_FF + n0 + r;
    rg[r] = F::load(G, row, lane, D_MODEL);
    ru[r] = F::load(Uq, row, lane, D_MODEL);
  }
  constexpr int P = 2 * NR * M;
  float v[P];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    typename F::U ug, uu;
    F::unpack(ug, rg[r], tsg);
    F::unpack(uu, ru[r], tsu);
#pragma unroll
    for (int t = 0; t < M; ++t) {
      v[r * M + t] = F::dot(ug, x[t]);
      v[NR * M + r * M + t] = F::dot(uu, x[t]);
    }
  }
  xreduce<P, 64>(v);
  // lanes < 32 hold gate sums, lane+32 the matching up sums
  const float u = __shfl_xor(v[0], 32);
  bool wr;
  const int idx = xreduce_index<P, 64>(lane, wr);
  if (lane < 32 && wr) {
    const int r = idx / M, t = idx % M;
    if (t < it.cnt) {
      const float h = silu_mul(v[0], u);
      uint16_t* hp = reinterpret_cast<uint16_t*>(a.h) + (size_t)row_of(a, it, t) * D_FF + n0 + r;
      if (OPER_F16<FMT>) *hp = (uint16_t)(pack_h16(h, 0.f) & 0xFFFFu);
      else *hp = f32_to_bf16(h);
    }
  }
}

// down: rows of 512; 16 lanes per row, a wave covers 4 rows per load and
// NRG such groups; lane owns chunk (lane & 15) of its row.
template <int FMT, int M, int NRG>
__device__ void gemv_down(const LayerArgs& a, const QMat& D, int mat, const ItemTok& it, int r0) {
  using F = GV<FMT>;
  const int lane = threadIdx.x & 63;
  const int chunk = lane & 15, rsub = lane >> 4;
  typename F::X x[M];
#pragma unroll
  for (int t = 0; t < M; ++t) {
    uint32_t src[16];
    if (t < it.cnt) {
      load_act<FMT>(src, reinterpret_cast<const uint16_t*>(a.h) + (size_t)row_of(a, it, t) * D_FF + 32 * chunk,
                    false);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) src[i] = 0u;
    }
    F::prep(x[t], src);
  }
  const float ts = (FMT == FMT_NVFP4) ? D.ts[mat] : 1.f;
  typename F::Raw rr[NRG];
#pragma unroll
  for (int g = 0; g < NRG; ++g) rr[g] = F::load(D, (size_t)mat * D_MODEL + r0 + 4 * g + rsub, chunk, D_FF);
  constexpr int P = NRG * M;
  float v[P];
#pragma unroll
  for (int g = 0; g < NRG; ++g) {
    typename F::U u;
    F::unpack(u, rr[g], ts);
#pragma unroll
    for (int t = 0; t < M; ++t) v[g * M + t] = F::dot(u, x[t]);
  }
  xreduce<P, 16>(v);
  bool wr;
  const int idx = xreduce_index<P, 16>(lane & 15, wr);
  if (wr) {
    const int g = idx / M, t = idx % M;
    if (t < it.cnt) a.y[(size_t)row_of(a, it, t) * D_MODEL + r0 + 4 * g + rsub] = v[0];
  }
}

// ======================================================================================
// MFMA items: weight tile of 128 rows x 64 k decoded into LDS, activation tile of
// 64 tokens x 64 k staged into LDS, v_mfma_f32_32x32x16_{f16,bf16}.
// ======================================================================================
constexpr int TS = 72;  // LDS row stride in 16-bit elements (64 + 8 pad)

struct MfmaSmem {
  uint16_t w[128 * TS];
  uint16_t x[MFMA_BN * TS];
  int tok[MFMA_BN];
  int row[MFMA_BN];
};

// Decode 32 consecutive weights (k0 .. k0+31 of one row) into 16 dwords of
// operand pairs, in the order the activation tile uses for this format.
template <int FMT> __device__ inline void mfma_decode_row32(const QMat& q, size_t row, int k0, int cols, uint32_t* o);

template <> __device__ inline void mfma_decode_row32<FMT_Q4_1>(const QMat& q, size_t row, int k0, int cols,
                                                               uint32_t* o) {
  const u32x4 c = ld16(q.codes + row * (cols / 2) + k0 / 2);
  const uint32_t dm = reinterpret_cast<const uint32_t*>(q.scales)[row * (cols / 32) + k0 / 32];
  const f16x2 d2 = {as_f16x2(dm)[0], as_f16x2(dm)[0]};
  const f16x2 m2 = {as_f16x2(dm)[1], as_f16x2(dm)[1]};
  const f16x2 off = {(_Float16)(-1024.f), (_Float16)(-1024.f)};
  const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // s = 0..3 -> pairs (q_s, q_{s+4}) of this 8-element group
      const uint32_t bits = ((w[j] >> (4 * s)) & 0x000F000Fu) | MAGIC;
      const f16x2 qv = as_f16x2(bits) + off;                  // exact small integers
      o[4 * j + s] = as_u32(__builtin_elementwise_fma(qv, d2, m2));  // fp16(d*q + m), one rounding
    }
  }
}

template <> __device__ inline void mfma_decode_row32<FMT_NVFP4>(const QMat& q, size_t row, int k0, int cols,
                                                                uint32_t* o) {
  const u32x4 c = ld16(q.codes + row * (cols / 2) + k0 / 2);
  const uint32_t sb = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(q.scales) +
                                                         row * (cols / 16) + k0 / 16);
  const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sb, 0);
  const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sb, 1);
  const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2 s = (j < 2) ? f16x2{s0, s0} : f16x2{s1, s1};
    o[4 * j + 0] = as_u32(as_f16x2(fp4x2_to_f16x2<0>(w[j])) * s);
    o[4 * j + 1] = as_u32(as_f16x2(fp4x2_to_f16x2<1>(w[j])) * s);
    o[4 * j + 2] = as_u32(as_f16x2(fp4x2_to_f16x2<2>(w[j])) * s);
    o[4 * j + 3] = as_u32(as_f16x2(fp4x2_to_f16x2<3>(w[j])) * s);
  }
}

template <> __device__ inline void mfma_decode_row32<FMT_BF16>(const QMat& q, size_t row, int k0, int cols,
                                                               uint32_t* o) {
  const uint8_t* p = q.codes + (row * cols + k0) * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = ld16(p + 16 * i);
    o[4 * i] = v[0]; o[4 * i + 1] = v[1]; o[4 * i + 2] = v[2]; o[4 * i + 3] = v[3];
  }
}

// Stage 16 activation elements (natural order pairs in src[8]) into LDS in the
// format's k order.
template <int FMT> __device__ inline void stage_x16(uint16_t* dst, const uint32_t* src) {
  uint32_t o[8];
  if (FMT == FMT_Q4_1) {
    q4_order(src[0], src[1], src[2], src[3], o);
    q4_order(src[4], src[5], src[6], src[7], o + 4);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = src[i];
  }
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(o[0], o[1], o[2], o[3]);
  d[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int FMT>
__device__ inline f32x16 mfma32(const uint16_t* a, const uint16_t* b, f32x16 c) {
  const uint4 av = *reinterpret_cast<const uint4*>(a);
  const uint4 bv = *reinterpret_cast<const uint4*>(b);
  if (OPER_F16<FMT>)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c, 0,
                                                  0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0,
                                                 0, 0);
}

// Fill the item's token/row tables in LDS (threads 0..63).
__device__ inline void mfma_tables(const LayerArgs& a, const ItemTok& it, MfmaSmem& sm) {
  const int i = threadIdx.x;
  if (i < MFMA_BN) {
    sm.tok[i] = (i < it.cnt) ? tok_of(a, it, i) : -1;
    sm.row[i] = (i < it.cnt) ? row_of(a, it, i) : -1;
  }
}

// gate/up item: 64 row pairs (n0 ..) x 64 tokens; LDS w rows 0..63 gate, 64..127 up.
template <int FMT>
__device__ void mfma_up(const LayerArgs& a, const QMat& G, const QMat& Uq, int mat, const ItemTok& it, int n0,
                        MfmaSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  mfma_tables(a, it, sm);
  __syncthreads();
  f32x16 acc[2] = {};
  // staging roles
  const int wr_row = tid >> 1, wr_half = tid & 1;  // 128 rows x 2 blocks of 32
  const QMat& wq = (wr_row < 64) ? G : Uq;
  const size_t wrow = (size_t)mat * D_FF + n0 + (wr_row & 63);
  const int xt = tid >> 2, xs = tid & 3;           // 64 tokens x 4 parts of 16
  const int xtok = sm.tok[xt];
  // MFMA roles: A-row r -> LDS row (r < 16 ? 16w + r : 64 + 16w + r - 16)
  const int ar = lane & 31;
  const int arow = (ar < 16) ? (16 * wave + ar) : (64 + 16 * wave + ar - 16);
  const int kh = 8 * (lane >> 5);
  for (int kc = 0; kc < D_MODEL; kc += 64) {
    uint32_t wv[16];
    mfma_decode_row32<FMT>(wq, wrow, kc + 32 * wr_half, D_MODEL, wv);
    uint32_t xv[8];
    if (xtok >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(a.x + (size_t)xtok * D_MODEL + kc + 16 * xs);
      const uint4 v0 = p[0], v1 = p[1];
      xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w; xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
      if (OPER_F16<FMT>) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = bf16x2_to_f16x2(xv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = 0u;
    }
    __syncthreads();  // previous chunk's MFMAs are done with the tiles
    {
      uint4* d = reinterpret_cast<uint4*>(sm.w + wr_row * TS + 32 * wr_half);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
      stage_x16<FMT>(sm.x + xt * TS + 16 * xs, xv);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint16_t* ap = sm.w + arow * TS + 16 * s + kh;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        acc[tt] = mfma32<FMT>(ap, sm.x + (32 * tt + ar) * TS + 16 * s + kh, acc[tt]);
    }
  }
  // epilogue: acc[tt][4i+j] = A-row 8i + 4(lane/32) + j, token 32tt + lane%32.
  // A-rows 0..15 gate, 16..31 up of the same n: gate i in {0,1}, up i+2.
  const float tsg = (FMT == FMT_NVFP4) ? G.ts[mat] : 1.f;
  const float tsu = (FMT == FMT_NVFP4) ? Uq.ts[mat] : 1.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int ti = 32 * tt + (lane & 31);
    const int hrow = sm.row[ti];
    if (hrow < 0) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = silu_mul(acc[tt][4 * i + j] * tsg, acc[tt][4 * (i + 2) + j] * tsu);
      const int n = n0 + 16 * wave + 8 * i + 4 * (lane >> 5);
      uint2 pk;
      if (OPER_F16<FMT>) { pk.x = pack_h16(hv[0], hv[1]); pk.y = pack_h16(hv[2], hv[3]); }
      else { pk.x = pack_b16(hv[0], hv[1]); pk.y = pack_b16(hv[2], hv[3]); }
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + (size_t)hrow * D_FF + n) = pk;
    }
  }
  __syncthreads();  // tables/tiles reused by the next item
}

// down item: 128 rows (r0 ..) x 64 tokens, K = 512.
template <int FMT>
__device__ void mfma_down(const LayerArgs& a, const QMat& D, int mat, const ItemTok& it, int r0, MfmaSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  mfma_tables(a, it, sm);
  __syncthreads();
  f32x16 acc[2] = {};
  const int wr_row = tid >> 1, wr_half = tid & 1;
  const size_t wrow = (size_t)mat * D_MODEL + r0 + wr_row;
  const int xt = tid >> 2, xs = tid & 3;
  const int xrow = sm.row[xt];
  const int ar = lane & 31;
  const int arow = 32 * wave + ar;
  const int kh = 8 * (lane >> 5);
  for (int kc = 0; kc < D_FF; kc += 64) {
    uint32_t wv[16];
    mfma_decode_row32<FMT>(D, wrow, kc + 32 * wr_half, D_FF, wv);
    uint32_t xv[8];
    if (xrow >= 0) {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.h) + (size_t)xrow * D_FF +
                                                      kc + 16 * xs);
      const uint4 v0 = p[0], v1 = p[1];
      xv[0] = v0.x; xv[1] = v0.y; xv[2] = v0.z; xv[3] = v0.w; xv[4] = v1.x; xv[5] = v1.y; xv[6] = v1.z; xv[7] = v1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = 0u;
    }
    __syncthreads();
    {
      uint4* d = reinterpret_cast<uint4*>(sm.w + wr_row * TS + 32 * wr_half);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
      stage_x16<FMT>(sm.x + xt * TS + 16 * xs, xv);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint16_t* ap = sm.w + arow * TS + 16 * s + kh;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        acc[tt] = mfma32<FMT>(ap, sm.x + (32 * tt + ar) * TS + 16 * s + kh, acc[tt]);
    }
  }
  const float ts = (FMT == FMT_NVFP4) ? D.ts[mat] : 1.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int ti = 32 * tt + (lane & 31);
    const int yrow = sm.row[ti];
    if (yrow < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 32 * wave + 8 * i + 4 * (lane >> 5);
      float4 o = make_float4(acc[tt][4 * i] * ts, acc[tt][4 * i + 1] * ts, acc[tt][4 * i + 2] * ts,
                             acc[tt][4 * i + 3] * ts);
      *reinterpret_cast<float4*>(a.y + (size_t)yrow * D_MODEL + r) = o;
    }
  }
  __syncthreads();
}

// ======================================================================================
// Persistent kernels
// ======================================================================================
template <int FMT> constexpr int UP_NR = (FMT == FMT_BF16) ? 2 : 4;   // row pairs per wave per step
template <int FMT> constexpr int DN_NRG = (FMT == FMT_BF16) ? 2 : 4;  // 4-row groups per wave per step

template <int FMT>
__global__ __launch_bounds__(256) void ffn_up_kernel(LayerArgs a) {
  __shared__ MfmaSmem sm;
  const int n_items = a.ctl[CTL_N_UP];
  const int wave = threadIdx.x >> 6;
  for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
    const uint32_t item = a.items_up[i];
    const int e = item_expert(item);
    const bool shared = e >= a.E;
    const QMat& G = shared ? a.sh_gate : a.gate;
    const QMat& U = shared ? a.sh_up : a.up;
    const int mat = shared ? 0 : e;
    const ItemTok it = item_tokens(a, e, item_tile(item));
    if (item_mfma(item)) {
      mfma_up<FMT>(a, G, U, mat, it, item_chunk(item) * UP_MFMA_ROWS, sm);
    } else {
      constexpr int NR = UP_NR<FMT>;
      // an item covers UP_GEMV_ROWS row pairs: 4 waves x (UP_GEMV_ROWS/4) rows, NR per step
      for (int r = 0; r < UP_GEMV_ROWS / 4; r += NR) {
        const int n0 = item_chunk(item) * UP_GEMV_ROWS + wave * (UP_GEMV_ROWS / 4) + r;
        if (it.cnt <= 1) gemv_up<FMT, 1, NR>(a, G, U, mat, it, n0);
        else if (it.cnt <= 2) gemv_up<FMT, 2, NR>(a, G, U, mat, it, n0);
        else gemv_up<FMT, 4, NR>(a, G, U, mat, it, n0);
      }
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void ffn_down_kernel(LayerArgs a) {
  __shared__ MfmaSmem sm;
  const int n_items = a.ctl[CTL_N_DN];
  const int wave = threadIdx.x >> 6;
  for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
    const uint32_t item = a.items_dn[i];
    const int e = item_expert(item);
    const bool shared = e >= a.E;
    const QMat& D = shared ? a.sh_down : a.down;
    const int mat = shared ? 0 : e;
    const ItemTok it = item_tokens(a, e, item_tile(item));
    if (item_mfma(item)) {
      mfma_down<FMT>(a, D, mat, it, item_chunk(item) * DN_MFMA_ROWS, sm);
    } else {
      constexpr int NRG = DN_NRG<FMT>;
      for (int g = 0; g < DN_GEMV_ROWS / 16; g += NRG) {
        const int r0 = item_chunk(item) * DN_GEMV_ROWS + wave * (DN_GEMV_ROWS / 4) + 4 * g;
        if (it.cnt <= 1) gemv_down<FMT, 1, NRG>(a, D, mat, it, r0);
        else if (it.cnt <= 2) gemv_down<FMT, 2, NRG>(a, D, mat, it, r0);
        else gemv_down<FMT, 4, NRG>(a, D, mat, it, r0);
      }
    }
  }
}

hipError_t launch_ffn_up(const LayerArgs& a, int grid, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: hipLaunchKernelGGL(ffn_up_kernel<FMT_Q4_1>, dim3(grid), dim3(256), 0, s, a); break;
    case FMT_NVFP4: hipLaunchKernelGGL(ffn_up_kernel<FMT_NVFP4>, dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(ffn_up_kernel<FMT_BF16>, dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_down(const LayerArgs& a, int grid, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: hipLaunchKernelGGL(ffn_down_kernel<FMT_Q4_1>, dim3(grid), dim3(256), 0, s, a); break;
    case FMT_NVFP4: hipLaunchKernelGGL(ffn_down_kernel<FMT_NVFP4>, dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(ffn_down_kernel<FMT_BF16>, dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
