// Expert FFN over the buckets: gate/up projection with fused SwiGLU, down
// projection with the weighted combine fused into its epilogue, and the
// residual/RMSNorm glue of stacked layers.
//
// The review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", argues that decoding
// this model is a weight-movement problem: each token touches 6 routed experts
// and the shared one out of 257 per layer.  So the work is organised around
// streaming each touched expert's packed weights from HBM once:
//   * buckets below MFMA_MIN tokens run on the vector ALUs in token groups of
//     up to 4 (two per pass): a lane owns one 32-element chunk of a weight row
//     (16 bytes of 4-bit codes), decodes it in registers to fp16 pairs and uses
//     v_dot2; each wave keeps a ring of row loads in flight and sums across
//     lanes with permlane swaps and DPP moves;
//   * buckets of MFMA_MIN or more tokens run on the matrix cores: a weight
//     tile is decoded into LDS once per 64-token tile (v_mfma 32x32x16), with
//     the next K-chunk prefetched into registers during the MFMAs.
// Both kernels are persistent and walk device-side work lists, so no host
// synchronisation is needed.  The shared expert does not depend on routing and
// runs as its own launches (on a second stream, overlapping the router).
//
// Combine: a separate kernel sums, per token, the K weighted expert rows in
// the fixed order j = 0..K-1 and the shared expert row, and rounds once to
// bf16 (in a stack it also updates the fp32 residual and writes the next
// layer's RMSNorm input).
#include "common.hpp"

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads: streaming (read once, non-temporal hint) or cached.
template <bool NT> __device__ inline u32x4 ld16(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT> __device__ inline uint32_t ld4(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  return *reinterpret_cast<const uint32_t*>(p);
}
template <bool NT> __device__ inline uint32_t ld2(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
  return *reinterpret_cast<const uint16_t*>(p);
}

constexpr uint32_t MAGIC = 0x64006400u;  // fp16 pair (1024, 1024): ORing a nibble into the
                                         // low mantissa bits gives 1024 + q exactly

// (w & mask) | magic in one v_and_or_b32.  gfx950 VOP3 takes no literal
// operands, so the mask rides in an SGPR and the magic in a VGPR; left to
// itself the compiler splits this into an AND and an OR.
__device__ inline uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic_v) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic_v));
  return r;
}

__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

__device__ inline float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_f16x2(a), as_f16x2(b), c, false);
}
__device__ inline float dot2b(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// E2M1 pair (byte B of w) -> fp16 pair, unscaled (exact).
template <int B> __device__ inline uint32_t fp4x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

// two bf16 (lo, hi halves of v) -> packed fp16 pair (exact for normal-range values)
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16), __uint_as_float(v & 0xFFFF0000u)));
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

// fp32 -> stored SwiGLU element: fp16 (saturated) for the 4-bit formats, bf16 otherwise.
template <int FMT> __device__ inline uint16_t h_store(float v);
template <> __device__ inline uint16_t h_store<FMT_Q4_1>(float v) {
  v = fminf(fmaxf(v, -65504.f), 65504.f);
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <> __device__ inline uint16_t h_store<FMT_NVFP4>(float v) { return h_store<FMT_Q4_1>(v); }
template <> __device__ inline uint16_t h_store<FMT_BF16>(float v) { return f32_to_bf16(v); }

// Operand precision of the expert GEMMs: fp16 for the 4-bit formats (their
// decoded values are exact in fp16), bf16 for bf16 weights.
template <int FMT> constexpr bool OPER_F16 = FMT != FMT_BF16;

// ======================================================================================
// Per-format chunk of a weight row: 32 consecutive elements owned by one lane.
// ======================================================================================
template <int FMT> struct GV;

template <> struct GV<FMT_Q4_1> {
  struct Raw { u32x4 c; uint32_t dm; };                // 16 B codes + fp16 {d, m}
  struct X { uint32_t p[16]; float se, so; };          // fp16 pairs in nibble order + even/odd sums
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    // row terms are workgroup-uniform; the unsigned lane terms let the loads
    // take the scalar-base + 32-bit vector-offset form
    r.c = ld16<NT>(q.codes + row * (cols / 2) + (sub * (uint32_t)(cols / 2) + 16u * (uint32_t)chunk));
    r.dm = ld4<NT>(reinterpret_cast<const uint32_t*>(q.scales) + row * (cols / 32) +
                   (sub * (uint32_t)(cols / 32) + (uint32_t)chunk));
    return r;
  }
  static __device__ void prep(X& x, const uint32_t* src) {  // src: 16 fp16 pairs, natural order
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
  // out[t] = sum_i w_i x_t,i over the chunk.  With the nibbles ORed into the
  // mantissa of 1024: lo = sum_even (1024+q) x, hi = sum_odd (1024+16q) x, so
  // the block dot d*sum q x + m*sum x = d lo + (d/16) hi + (m-1024d) se + (m-64d) so.
  template <int M> static __device__ void dot(const Raw& r, const X* x, float* out, float) {
    float lo[M], hi[M];
#pragma unroll
    for (int t = 0; t < M; ++t) { lo[t] = 0.f; hi[t] = 0.f; }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = r.c[j], w8 = w >> 8;
      const uint32_t A = (w & 0x000F000Fu) | MAGIC, B = (w & 0x00F000F0u) | MAGIC;
      const uint32_t C = (w8 & 0x000F000Fu) | MAGIC, D = (w8 & 0x00F000F0u) | MAGIC;
#pragma unroll
      for (int t = 0; t < M; ++t) {
        lo[t] = dot2h(A, x[t].p[4 * j + 0], lo[t]);
        hi[t] = dot2h(B, x[t].p[4 * j + 1], hi[t]);
        lo[t] = dot2h(C, x[t].p[4 * j + 2], lo[t]);
        hi[t] = dot2h(D, x[t].p[4 * j + 3], hi[t]);
      }
    }
    const float d = f16lo(r.dm), m = f16hi(r.dm);
    const float c2 = d * 0.0625f, c3 = m - 1024.f * d, c4 = m - 64.f * d;
#pragma unroll
    for (int t = 0; t < M; ++t) out[t] = d * lo[t] + c2 * hi[t] + c3 * x[t].se + c4 * x[t].so;
  }
  // single-token form: nibbles unpacked once per row, then one dot per token
  struct U { uint32_t A[4], B[4], C[4], D[4]; float d, c2, c3, c4; };
  static __device__ void unpack(U& u, const Raw& r, float) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = r.c[j], w8 = w >> 8;
      u.A[j] = and_or(w, 0x000F000Fu, MAGIC);
      u.B[j] = and_or(w, 0x00F000F0u, MAGIC);
      u.C[j] = and_or(w8, 0x000F000Fu, MAGIC);
      u.D[j] = and_or(w8, 0x00F000F0u, MAGIC);
    }
    const float d = f16lo(r.dm), m = f16hi(r.dm);
    u.d = d;
    u.c2 = d * 0.0625f;
    u.c3 = m - 1024.f * d;
    u.c4 = m - 64.f * d;
  }
  static __device__ float dot1(const U& u, const X& x) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo = dot2h(u.A[j], x.p[4 * j + 0], lo);
      hi = dot2h(u.B[j], x.p[4 * j + 1], hi);
      lo = dot2h(u.C[j], x.p[4 * j + 2], lo);
      hi = dot2h(u.D[j], x.p[4 * j + 3], hi);
    }
    return u.d * lo + u.c2 * hi + u.c3 * x.se + u.c4 * x.so;
  }
  // even/odd sums of a chunk stored in nibble order: pairs 0 and 2 of each group
  // of four hold even elements, pairs 1 and 3 odd ones
  static __device__ void sums(X& x) {
    float se = 0.f, so = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      se += f16lo(x.p[4 * j]) + f16hi(x.p[4 * j]) + f16lo(x.p[4 * j + 2]) + f16hi(x.p[4 * j + 2]);
      so += f16lo(x.p[4 * j + 1]) + f16hi(x.p[4 * j + 1]) + f16lo(x.p[4 * j + 3]) + f16hi(x.p[4 * j + 3]);
    }
    x.se = se;
    x.so = so;
  }
  // 32 decoded weights as 16 fp16 pairs in nibble order (matrix-core path):
  // fp16(d*q + m), rounded once.
  static __device__ void decode(const Raw& r, uint32_t* o) {
    const f16x2 d2 = {as_f16x2(r.dm)[0], as_f16x2(r.dm)[0]};
    const f16x2 m2 = {as_f16x2(r.dm)[1], as_f16x2(r.dm)[1]};
    const f16x2 off = {(_Float16)(-1024.f), (_Float16)(-1024.f)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t bits = ((r.c[j] >> (4 * s)) & 0x000F000Fu) | MAGIC;  // (q_s, q_{s+4})
        const f16x2 qv = as_f16x2(bits) + off;                             // exact small integers
        o[4 * j + s] = as_u32(__builtin_elementwise_fma(qv, d2, m2));
      }
    }
  }
};

template <> struct GV<FMT_NVFP4> {
  struct Raw { u32x4 c; uint32_t s; };                 // 16 B codes + 2 E4M3 block scales
  struct X { uint32_t p[16]; };                        // fp16 pairs, natural order
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    r.c = ld16<NT>(q.codes + row * (cols / 2) + (sub * (uint32_t)(cols / 2) + 16u * (uint32_t)chunk));
    r.s = ld2<NT>(reinterpret_cast<const uint8_t*>(q.scales) + row * (cols / 16) +
                  (sub * (uint32_t)(cols / 16) + 2u * (uint32_t)chunk));
    return r;
  }
  static __device__ void prep(X& x, const uint32_t* src) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x.p[i] = src[i];
  }
  template <int M> static __device__ void dot(const Raw& r, const X* x, float* out, float ts) {
    float a0[M], a1[M];
#pragma unroll
    for (int t = 0; t < M; ++t) { a0[t] = 0.f; a1[t] = 0.f; }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = r.c[j];
      const uint32_t P0 = fp4x2_to_f16x2<0>(w), P1 = fp4x2_to_f16x2<1>(w);
      const uint32_t P2 = fp4x2_to_f16x2<2>(w), P3 = fp4x2_to_f16x2<3>(w);
#pragma unroll
      for (int t = 0; t < M; ++t) {
        float& acc = (j < 2) ? a0[t] : a1[t];
        acc = dot2h(P0, x[t].p[4 * j + 0], acc);
        acc = dot2h(P1, x[t].p[4 * j + 1], acc);
        acc = dot2h(P2, x[t].p[4 * j + 2], acc);
        acc = dot2h(P3, x[t].p[4 * j + 3], acc);
      }
    }
    const float s0 = __builtin_amdgcn_cvt_f32_fp8(r.s, 0) * ts;
    const float s1 = __builtin_amdgcn_cvt_f32_fp8(r.s, 1) * ts;
#pragma unroll
    for (int t = 0; t < M; ++t) out[t] = s0 * a0[t] + s1 * a1[t];
  }
  struct U { uint32_t P[16]; float s0, s1; };
  static __device__ void unpack(U& u, const Raw& r, float ts) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u.P[4 * j + 0] = fp4x2_to_f16x2<0>(r.c[j]);
      u.P[4 * j + 1] = fp4x2_to_f16x2<1>(r.c[j]);
      u.P[4 * j + 2] = fp4x2_to_f16x2<2>(r.c[j]);
      u.P[4 * j + 3] = fp4x2_to_f16x2<3>(r.c[j]);
    }
    u.s0 = __builtin_amdgcn_cvt_f32_fp8(r.s, 0) * ts;
    u.s1 = __builtin_amdgcn_cvt_f32_fp8(r.s, 1) * ts;
  }
  static __device__ float dot1(const U& u, const X& x) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a0 = dot2h(u.P[i], x.p[i], a0);
#pragma unroll
    for (int i = 8; i < 16; ++i) a1 = dot2h(u.P[i], x.p[i], a1);
    return u.s0 * a0 + u.s1 * a1;
  }
  static __device__ void sums(X&) {}
  // E2M1 * E4M3 is exact in fp16; the per-matrix scale is applied after the MFMA.
  static __device__ void decode(const Raw& r, uint32_t* o) {
    const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(r.s, 0);
    const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(r.s, 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2 s = (j < 2) ? f16x2{s0, s0} : f16x2{s1, s1};
      o[4 * j + 0] = as_u32(as_f16x2(fp4x2_to_f16x2<0>(r.c[j])) * s);
      o[4 * j + 1] = as_u32(as_f16x2(fp4x2_to_f16x2<1>(r.c[j])) * s);
      o[4 * j + 2] = as_u32(as_f16x2(fp4x2_to_f16x2<2>(r.c[j])) * s);
      o[4 * j + 3] = as_u32(as_f16x2(fp4x2_to_f16x2<3>(r.c[j])) * s);
    }
  }
};

template <> struct GV<FMT_BF16> {
  struct Raw { u32x4 c[4]; };                          // 64 B of bf16
  struct X { uint32_t p[16]; };                        // bf16 pairs, natural order
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    const uint8_t* p = q.codes + row * cols * 2 + (sub * (uint32_t)(cols * 2) + 64u * (uint32_t)chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = ld16<NT>(p + 16 * i);
    return r;
  }
  static __device__ void prep(X& x, const uint32_t* src) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x.p[i] = src[i];
  }
  template <int M> static __device__ void dot(const Raw& r, const X* x, float* out, float) {
#pragma unroll
    for (int t = 0; t < M; ++t) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) a = dot2b(r.c[i >> 2][i & 3], x[t].p[i], a);
      out[t] = a;
    }
  }
  struct U { uint32_t P[16]; };
  static __device__ void unpack(U& u, const Raw& r, float) {
#pragma unroll
    for (int i = 0; i < 16; ++i) u.P[i] = r.c[i >> 2][i & 3];
  }
  static __device__ float dot1(const U& u, const X& x) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = dot2b(u.P[i], x.p[i], a);
    return a;
  }
  static __device__ void sums(X&) {}
  static __device__ void decode(const Raw& r, uint32_t* o) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = r.c[i >> 2][i & 3];
  }
};

// 32 activation elements of one lane as 16 operand pairs, natural order.  src
// points at bf16 (x) or at the stored SwiGLU output (already operand typed).
template <int FMT> __device__ inline void load_act(uint32_t* d, const uint16_t* src, bool src_bf16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = ld16<false>(src + 8 * i);
    d[4 * i] = v[0]; d[4 * i + 1] = v[1]; d[4 * i + 2] = v[2]; d[4 * i + 3] = v[3];
  }
  if (OPER_F16<FMT> && src_bf16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) d[i] = bf16x2_to_f16x2(d[i]);
  }
}

// Lane exchange for reduction step `m` (partner lane = lane ^ m, except m = 4
// which pairs lane i with 7 - i inside each group of 8).  Steps 32 and 16 use
// the gfx950 permlane swaps: swap(a, b).x + .y holds a's pair sum in the lanes
// whose bit m is clear and b's pair sum in the others.  Steps below 16 use DPP.
template <int M> __device__ inline float dpp_partner(float v) {
  constexpr int ctrl = (M == 8) ? 0x128 : (M == 4) ? 0x141 : (M == 2) ? 0x4E : 0xB1;  // ror8, half-mirror, quad perms
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}
template <int M> __device__ inline float halve_step(float a, float b) {
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const bool hi = (threadIdx.x & M) != 0;
    const float sa = a + dpp_partner<M>(a), sb = b + dpp_partner<M>(b);
    return hi ? sb : sa;
  }
}
template <int M> __device__ inline float plain_step(float a) { return halve_step<M>(a, a); }

// Transposing reduction: P partials per lane, summed over groups of G lanes
// (steps G/2 .. 1).  While more than one value is left, each step halves the
// count: lanes with bit m clear keep the first half, the others the second.
// Afterwards v[0] of a lane holds the total of index
// idx(lane) = sum over halving steps s of bit(lane, G >> (s+1)) * P >> (s+1).
template <int P, int G, int M = G / 2>
__device__ inline void xreduce(float* v) {
  if constexpr (M >= 1) {
    if constexpr (P > 1) {
#pragma unroll
      for (int i = 0; i < P / 2; ++i) v[i] = halve_step<M>(v[i], v[i + P / 2]);
      xreduce<P / 2, G, M / 2>(v);
    } else {
      v[0] = plain_step<M>(v[0]);
      xreduce<1, G, M / 2>(v);
    }
  }
}

// Index a lane holds after xreduce<P, G>, and whether it is the lane of its
// group that writes it (the bits of the non-halving steps are zero).
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

// Tokens of an item: bucket positions p0 .. p0+cnt-1 of a routed expert
// (expert-output row p), or tokens p0 .. p0+cnt-1 of the shared expert
// (expert-output row S + t).  Vector-path items carry their token ids.
struct ItemTok {
  int p0, cnt;
  bool shared, mfma;
  int tok[GV_GROUP];
};

__device__ inline ItemTok item_tokens(const Item& item, bool shared) {
  ItemTok r;
  r.shared = shared;
  r.mfma = item_mfma(item.head);
  r.p0 = (int)item.p0;
  r.cnt = item_count(item.head);
  r.tok[0] = (int)(item.t01 & 0xFFFFu);
  r.tok[1] = (int)(item.t01 >> 16);
  r.tok[2] = (int)(item.t23 & 0xFFFFu);
  r.tok[3] = (int)(item.t23 >> 16);
  return r;
}
// token of entry i: shared -> p0 + i; vector path -> carried id; matrix path -> perm
__device__ inline int tok_of(const LayerArgs& a, const ItemTok& it, int i) {
  if (it.shared) return it.p0 + i;
  if (!it.mfma) return it.tok[i];
  return a.perm[it.p0 + i] / a.K;
}
__device__ inline int row_of(const LayerArgs& a, const ItemTok& it, int i) {
  return it.shared ? a.S + it.p0 + i : it.p0 + i;
}

// Shared-expert items are implicit: item i -> tile i / chunks, chunk i % chunks.
__device__ inline Item shared_item(int T, int E, int i, int chunks) {
  const bool mf = bucket_mfma(T);
  const int per = mf ? MFMA_BN : GV_GROUP;
  const int tile = i / chunks;
  Item it;
  it.p0 = (uint32_t)(tile * per);
  it.head = item_head(E, i % chunks, min(per, T - tile * per), mf);
  it.t01 = it.p0 | ((it.p0 + 1) << 16);
  it.t23 = (it.p0 + 2) | ((it.p0 + 3) << 16);
  return it;
}
__device__ inline int shared_items(int T, int chunks) { return bucket_tiles(T) * chunks; }

// ======================================================================================
// Vector-path items
// ======================================================================================

// ======================================================================================
// Vector path as a continuous stream.  A persistent workgroup walks its chunks
// c, c + G, c + 2G, ... (G = grid size).  A chunk is one token group (<= 4
// tokens) of one expert times UP_ROWS row pairs (gate/up) or DN_ROWS rows
// (down); each wave owns a fixed quarter of the chunk's rows.  The activations
// of the chunk's tokens sit in LDS (double buffered: the next chunk's are
// loaded during this one), and every wave keeps a ring of weight-row loads in
// flight that runs on into the next chunk, so the weight stream never drains
// between chunks.
// ======================================================================================
template <int FMT> constexpr int UP_RING = (FMT == FMT_BF16) ? 2 : 4;  // row pairs in flight per wave
template <int FMT> constexpr int DN_RING = (FMT == FMT_BF16) ? 4 : 8;  // 4-row groups in flight per wave
constexpr int UP_STEPS = UP_ROWS / 4;        // row pairs per wave per chunk (16)
constexpr int DN_STEPS = DN_ROWS / 16;       // 4-row groups per wave per chunk (8)

// Activations of a chunk in LDS: [buffer][token][piece j][slot][16 B]; piece j
// of a slot holds elements 8j..8j+7 of that slot's 32-element chunk (already in
// the format's operand type and k order).  Gate/up: slot = lane (2048-long
// rows); down: slot = lane & 15 (512-long rows).
struct GvSmem {
  u32x4 x[2][GV_GROUP][4][64];
};

// Loads of one chunk's activations into registers: thread (slot = tid / 4,
// piece = tid % 4) takes 8 elements of each token (zeros for absent tokens).
struct XStage {
  u32x4 v[GV_GROUP];
};

template <int FMT, bool UP>
__device__ inline void xstage_load(const LayerArgs& a, const ItemTok& it, XStage& st) {
  const int tid = threadIdx.x;
  const int slot = tid >> 2, piece = tid & 3;
#pragma unroll
  for (int t = 0; t < GV_GROUP; ++t) {
    st.v[t] = u32x4{0u, 0u, 0u, 0u};
    if (t < it.cnt && (UP || slot < 16)) {
      const uint16_t* src = UP ? a.x + (size_t)tok_of(a, it, t) * D_MODEL + 32 * slot + 8 * piece
                               : a.h + (size_t)row_of(a, it, t) * D_FF + 32 * slot + 8 * piece;
      st.v[t] = ld16<false>(src);
    }
  }
}

template <int FMT, bool UP>
__device__ inline void xstage_store(const XStage& st, GvSmem& sm, int buf) {
  const int tid = threadIdx.x;
  const int slot = tid >> 2, piece = tid & 3;
  if (!UP && slot >= 16) return;
#pragma unroll
  for (int t = 0; t < GV_GROUP; ++t) {
    uint32_t n[4] = {st.v[t][0], st.v[t][1], st.v[t][2], st.v[t][3]};
    if (OPER_F16<FMT> && UP) {  // x arrives as bf16; the stored SwiGLU output is already operand typed
#pragma unroll
      for (int i = 0; i < 4; ++i) n[i] = bf16x2_to_f16x2(n[i]);
    }
    uint32_t o[4];
    if (FMT == FMT_Q4_1) {
      q4_order(n[0], n[1], n[2], n[3], o);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = n[i];
    }
    sm.x[buf][t][piece][slot] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int FMT>
__device__ inline void x_from_lds(typename GV<FMT>::X& x, const GvSmem& sm, int buf, int t, int slot) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = sm.x[buf][t][j][slot];
    x.p[4 * j] = v[0]; x.p[4 * j + 1] = v[1]; x.p[4 * j + 2] = v[2]; x.p[4 * j + 3] = v[3];
  }
}

// Weight matrices of a chunk's expert (uniform across the workgroup).
struct ChunkW {
  QMat g, u;   // gate/up (or the down matrix in g)
  int mat;
  float tsg, tsu;
};

template <int FMT, bool SHARED, bool UP>
__device__ inline ChunkW chunk_weights(const LayerArgs& a, const Item& item) {
  ChunkW w;
  const int e = SHARED ? 0 : item_expert(item.head);
  w.mat = e;
  if (UP) {
    w.g = SHARED ? a.sh_gate : a.gate;
    w.u = SHARED ? a.sh_up : a.up;
  } else {
    w.g = SHARED ? a.sh_down : a.down;
    w.u = w.g;
  }
  w.tsg = (FMT == FMT_NVFP4) ? w.g.ts[e] : 1.f;
  w.tsu = (FMT == FMT_NVFP4) ? w.u.ts[e] : 1.f;
  return w;
}

// The item of a chunk is the same for the whole workgroup: keep it in SGPRs so
// that the row addresses derived from it are scalar.
template <bool SHARED>
__device__ inline Item fetch_item(const LayerArgs& a, const Item* list, int idx, int chunks) {
  Item it = SHARED ? shared_item(a.T, a.E, idx, chunks) : list[idx];
  it.head = __builtin_amdgcn_readfirstlane(it.head);
  it.p0 = __builtin_amdgcn_readfirstlane(it.p0);
  it.t01 = __builtin_amdgcn_readfirstlane(it.t01);
  it.t23 = __builtin_amdgcn_readfirstlane(it.t23);
  return it;
}

template <int MT> constexpr int POW2_UP = MT <= 1 ? 1 : MT <= 2 ? 2 : MT <= 4 ? 4 : 8;

// value of lane ^ 32 in the lanes below 32
__device__ inline float upper_half(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}

// One chunk of gate/up for MT token slots (slots >= the item's count hold zero
// activations): UP_STEPS row pairs per wave from the ring, each slot refilled
// with the row UP_RING steps ahead, which past the chunk's end is a row of the
// next chunk (nw, nr0) when there is one.
template <int FMT, int MT>
__device__ inline void up_chunk(typename GV<FMT>::Raw* rg, typename GV<FMT>::Raw* ru, const ChunkW& w, size_t r0,
                                const ChunkW& nw, size_t nr0, bool has_next, const GvSmem& sm, int buf, int cnt,
                                uint16_t* hbase) {
  using F = GV<FMT>;
  constexpr int D = UP_RING<FMT>;
  constexpr int RP = POW2_UP<MT>;          // token slots padded to a power of two
  constexpr int EPI = 4 / RP;              // steps whose sums are reduced together (8 sums per lane)
  constexpr int P = 2 * EPI * RP;          // partial sums per lane: [gate/up][step][token]
  static_assert(UP_STEPS % EPI == 0 && P <= 64, "reduction batch");
  const int lane = threadIdx.x & 63;
  typename F::X xs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    x_from_lds<FMT>(xs[t], sm, buf, t, lane);
    F::sums(xs[t]);
  }
  // after the transposing reduction a lane holds one (gate/up, step, token)
  // total; the gate totals sit in lanes < 32 and the matching up totals in lane ^ 32
  bool wr;
  const int my_idx = xreduce_index<P, 64>(lane, wr);
  const int my_t = my_idx % RP, my_r = (my_idx / RP) % EPI;
  const bool writer = lane < 32 && wr && my_t < cnt;
  uint16_t* hdst = hbase + (size_t)my_t * D_FF + my_r;
  float v[P];
#pragma unroll
  for (int s = 0; s < UP_STEPS; ++s) {
    const int slot = s % D, r = s % EPI;
    typename F::U ug, uu;
    F::unpack(ug, rg[slot], w.tsg);
    F::unpack(uu, ru[slot], w.tsu);
    if (s + D < UP_STEPS) {
      rg[slot] = F::template load<true>(w.g, r0 + s + D, 0u, lane, D_MODEL);
      ru[slot] = F::template load<true>(w.u, r0 + s + D, 0u, lane, D_MODEL);
    } else if (has_next) {
      rg[slot] = F::template load<true>(nw.g, nr0 + s + D - UP_STEPS, 0u, lane, D_MODEL);
      ru[slot] = F::template load<true>(nw.u, nr0 + s + D - UP_STEPS, 0u, lane, D_MODEL);
    }
#pragma unroll
    for (int t = 0; t < RP; ++t) {
      v[r * RP + t] = (t < MT) ? F::dot1(ug, xs[t < MT ? t : 0]) : 0.f;
      v[(EPI + r) * RP + t] = (t < MT) ? F::dot1(uu, xs[t < MT ? t : 0]) : 0.f;
    }
    if (r == EPI - 1) {
      xreduce<P, 64>(v);
      const float u = upper_half(v[0]);
      if (writer) hdst[s - r] = h_store<FMT>(silu_mul(v[0], u));
    }
  }
}

// gate/up + SwiGLU over vector-path chunks [0, n) of `list` (or of the shared
// expert), this workgroup taking c = blockIdx.x, +gridDim.x, ...
template <int FMT, bool SHARED>
__device__ void up_stream(const LayerArgs& a, const Item* list, int n, GvSmem& sm) {
  using F = GV<FMT>;
  constexpr int D = UP_RING<FMT>;
  static_assert(UP_STEPS % D == 0, "ring must divide the steps of a chunk");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int c = blockIdx.x;
  if (c >= n) return;
  Item item = fetch_item<SHARED>(a, list, c, N_UP_CHUNKS);
  ItemTok it = item_tokens(item, SHARED);
  ChunkW w = chunk_weights<FMT, SHARED, true>(a, item);
  // this wave's row pairs of a chunk: first_row + s, s = 0 .. UP_STEPS-1
  auto first_row = [&](const Item& itm, const ChunkW& cw) {
    return (size_t)cw.mat * D_FF + item_chunk(itm.head) * UP_ROWS + wave * UP_STEPS;
  };
  size_t r0 = first_row(item, w);
  typename F::Raw rg[D], ru[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    rg[i] = F::template load<true>(w.g, r0 + i, 0u, lane, D_MODEL);
    ru[i] = F::template load<true>(w.u, r0 + i, 0u, lane, D_MODEL);
  }
  int buf = 0;
  {
    XStage st;
    xstage_load<FMT, true>(a, it, st);
    xstage_store<FMT, true>(st, sm, buf);
  }
  __syncthreads();
#pragma unroll 1
  for (;;) {
    const int nc = c + gridDim.x;
    const bool has_next = nc < n;
    Item nitem = item;
    ItemTok nit = it;
    ChunkW nw = w;
    size_t nr0 = r0;
    XStage st;
    if (has_next) {
      nitem = fetch_item<SHARED>(a, list, nc, N_UP_CHUNKS);
      nit = item_tokens(nitem, SHARED);
      nw = chunk_weights<FMT, SHARED, true>(a, nitem);
      nr0 = first_row(nitem, nw);
      xstage_load<FMT, true>(a, nit, st);
    }
    const int cnt = it.cnt;
    uint16_t* hbase = a.h + (size_t)row_of(a, it, 0) * D_FF + item_chunk(item.head) * UP_ROWS + wave * UP_STEPS;
    if (cnt <= 1) up_chunk<FMT, 1>(rg, ru, w, r0, nw, nr0, has_next, sm, buf, cnt, hbase);
    else if (cnt == 2) up_chunk<FMT, 2>(rg, ru, w, r0, nw, nr0, has_next, sm, buf, cnt, hbase);
    else if (cnt == 3) up_chunk<FMT, 3>(rg, ru, w, r0, nw, nr0, has_next, sm, buf, cnt, hbase);
    else up_chunk<FMT, GV_GROUP>(rg, ru, w, r0, nw, nr0, has_next, sm, buf, cnt, hbase);
    if (!has_next) break;
    xstage_store<FMT, true>(st, sm, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    c = nc;
    item = nitem;
    it = nit;
    w = nw;
    r0 = nr0;
  }
}

// One chunk of down for MT token slots: DN_STEPS groups of 4 rows per wave (16
// lanes per 512-long row), ring refilled as in up_chunk.
template <int FMT, int MT>
__device__ inline void down_chunk(typename GV<FMT>::Raw* ring, const ChunkW& w, size_t r0, const ChunkW& nw,
                                  size_t nr0, bool has_next, const GvSmem& sm, int buf, int cnt, float* ybase) {
  using F = GV<FMT>;
  constexpr int R = DN_RING<FMT> < DN_STEPS ? DN_RING<FMT> : DN_STEPS;
  constexpr int RP = POW2_UP<MT>;
  constexpr int EPI = 8 / RP;                              // row groups reduced together (8 sums per lane)
  constexpr int P = EPI * RP;                              // partial sums per lane: [group][token]
  static_assert(DN_STEPS % EPI == 0 && P <= 16, "reduction batch");
  const int slot16 = threadIdx.x & 15;
  const uint32_t sub = (threadIdx.x & 63) >> 4;  // row of the lane within a 4-row group
  typename F::X xs[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    x_from_lds<FMT>(xs[t], sm, buf, t, slot16);
    F::sums(xs[t]);
  }
  bool wr;
  const int my_idx = xreduce_index<P, 16>(slot16, wr);
  const int my_t = my_idx % RP, my_g = my_idx / RP;
  const bool writer = wr && my_t < cnt;
  float* ydst = ybase + (size_t)my_t * D_MODEL + 4 * my_g;
  float v[P];
#pragma unroll
  for (int g = 0; g < DN_STEPS; ++g) {
    const int slot = g % R, r = g % EPI;
    typename F::U u;
    F::unpack(u, ring[slot], w.tsg);
    if (g + R < DN_STEPS) {
      ring[slot] = F::template load<true>(w.g, r0 + 4 * (g + R), sub, slot16, D_FF);
    } else if (has_next) {
      ring[slot] = F::template load<true>(nw.g, nr0 + 4 * (g + R - DN_STEPS), sub, slot16, D_FF);
    }
#pragma unroll
    for (int t = 0; t < RP; ++t) v[r * RP + t] = (t < MT) ? F::dot1(u, xs[t < MT ? t : 0]) : 0.f;
    if (r == EPI - 1) {
      xreduce<P, 16>(v);
      if (writer) ydst[4 * (g - r)] = v[0];
    }
  }
}

// down over vector-path chunks, workgroup-strided as up_stream
template <int FMT, bool SHARED>
__device__ void down_stream(const LayerArgs& a, const Item* list, int n, GvSmem& sm) {
  using F = GV<FMT>;
  constexpr int R = DN_RING<FMT> < DN_STEPS ? DN_RING<FMT> : DN_STEPS;
  static_assert(DN_STEPS % R == 0, "ring must divide the steps of a chunk");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot16 = threadIdx.x & 15, rsub = (threadIdx.x & 63) >> 4;
  int c = blockIdx.x;
  if (c >= n) return;
  Item item = fetch_item<SHARED>(a, list, c, N_DN_CHUNKS);
  ItemTok it = item_tokens(item, SHARED);
  ChunkW w = chunk_weights<FMT, SHARED, false>(a, item);
  // rows of this lane: first_row + rsub + 4 g, g = 0 .. DN_STEPS-1 (first_row is
  // workgroup-uniform, rsub the lane's row within a 4-row group)
  auto first_row = [&](const Item& itm, const ChunkW& cw) {
    return (size_t)cw.mat * D_MODEL + item_chunk(itm.head) * DN_ROWS + wave * (DN_ROWS / 4);
  };
  size_t r0 = first_row(item, w);
  typename F::Raw ring[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ring[i] = F::template load<true>(w.g, r0 + 4 * i, (uint32_t)rsub, slot16, D_FF);
  int buf = 0;
  {
    XStage st;
    xstage_load<FMT, false>(a, it, st);
    xstage_store<FMT, false>(st, sm, buf);
  }
  __syncthreads();
#pragma unroll 1
  for (;;) {
    const int nc = c + gridDim.x;
    const bool has_next = nc < n;
    Item nitem = item;
    ItemTok nit = it;
    ChunkW nw = w;
    size_t nr0 = r0;
    XStage st;
    if (has_next) {
      nitem = fetch_item<SHARED>(a, list, nc, N_DN_CHUNKS);
      nit = item_tokens(nitem, SHARED);
      nw = chunk_weights<FMT, SHARED, false>(a, nitem);
      nr0 = first_row(nitem, nw);
      xstage_load<FMT, false>(a, nit, st);
    }
    const int cnt = it.cnt;
    float* ybase =
        a.y + (size_t)row_of(a, it, 0) * D_MODEL + item_chunk(item.head) * DN_ROWS + wave * (DN_ROWS / 4) + rsub;
    if (cnt <= 1) down_chunk<FMT, 1>(ring, w, r0, nw, nr0, has_next, sm, buf, cnt, ybase);
    else if (cnt == 2) down_chunk<FMT, 2>(ring, w, r0, nw, nr0, has_next, sm, buf, cnt, ybase);
    else if (cnt == 3) down_chunk<FMT, 3>(ring, w, r0, nw, nr0, has_next, sm, buf, cnt, ybase);
    else down_chunk<FMT, GV_GROUP>(ring, w, r0, nw, nr0, has_next, sm, buf, cnt, ybase);
    if (!has_next) break;
    xstage_store<FMT, false>(st, sm, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    c = nc;
    item = nitem;
    it = nit;
    w = nw;
    r0 = nr0;
  }
}

// ======================================================================================
// Matrix-core items: weight tile of 128 rows x 64 k decoded into LDS, activation
// tile of 64 tokens x 64 k staged into LDS, v_mfma_f32_32x32x16_{f16,bf16}; the
// next K-chunk is loaded into registers while the current one is multiplied.
// ======================================================================================
constexpr int TS = 72;  // LDS row stride in 16-bit elements (64 + 8 pad)

struct FfnSmem {
  uint16_t w[128 * TS];
  uint16_t x[MFMA_BN * TS];
  int tok[MFMA_BN];
  int row[MFMA_BN];
};

// Store 16 activation elements (natural-order pairs src[8]) into LDS in the
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
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  d[0] = u32x4{o[0], o[1], o[2], o[3]};
  d[1] = u32x4{o[4], o[5], o[6], o[7]};
}

template <int FMT>
__device__ inline f32x16 mfma32(const uint16_t* a, const uint16_t* b, f32x16 c) {
  const u32x4 av = *reinterpret_cast<const u32x4*>(a);
  const u32x4 bv = *reinterpret_cast<const u32x4*>(b);
  if (OPER_F16<FMT>)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c, 0,
                                                  0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0,
                                                 0, 0);
}

__device__ inline void mfma_tables(const LayerArgs& a, const ItemTok& it, FfnSmem& sm) {
  const int i = threadIdx.x;
  if (i < MFMA_BN) {
    // matrix-core tiles are shared-expert tiles or routed buckets (tokens via perm)
    sm.tok[i] = (i < it.cnt) ? (it.shared ? it.p0 + i : a.perm[it.p0 + i] / a.K) : -1;
    sm.row[i] = (i < it.cnt) ? row_of(a, it, i) : -1;
  }
}

// One K-chunk of a 128-row x 64-token tile: thread (wr_row = tid/2, half = tid%2)
// owns 32 weights of one row; thread (xt = tid/4, xs = tid%4) owns 16
// activation elements of one token.
template <int FMT> struct MfmaStage {
  typename GV<FMT>::Raw w;
  u32x4 x0, x1;
};

template <int FMT>
__device__ inline void mfma_fetch(MfmaStage<FMT>& st, const QMat& wq, size_t wrow, int kw, const uint16_t* xsrc,
                                  int cols) {
  st.w = GV<FMT>::template load<false>(wq, wrow, 0u, kw / 32, cols);
  if (xsrc) {
    st.x0 = ld16<false>(xsrc);
    st.x1 = ld16<false>(xsrc + 8);
  } else {
    st.x0 = u32x4{0u, 0u, 0u, 0u};
    st.x1 = st.x0;
  }
}

template <int FMT>
__device__ inline void mfma_stage_store(const MfmaStage<FMT>& st, FfnSmem& sm, int wr_row, int wr_half, int xt, int xs,
                                        bool x_bf16) {
  uint32_t wv[16];
  GV<FMT>::decode(st.w, wv);
  u32x4* d = reinterpret_cast<u32x4*>(sm.w + wr_row * TS + 32 * wr_half);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = u32x4{wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]};
  uint32_t xv[8] = {st.x0[0], st.x0[1], st.x0[2], st.x0[3], st.x1[0], st.x1[1], st.x1[2], st.x1[3]};
  if (OPER_F16<FMT> && x_bf16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = bf16x2_to_f16x2(xv[i]);
  }
  stage_x16<FMT>(sm.x + xt * TS + 16 * xs, xv);
}

// acc[tt] += W_tile(rows arow..) x X_tile(tokens 32tt..) over K = kdim.
// wq/wrow: this thread's weight row; xrow_ptr: this thread's activation row (or null).
template <int FMT>
__device__ inline void mfma_kloop(f32x16* acc, FfnSmem& sm, const QMat& wq, size_t wrow, const uint16_t* xrow_ptr,
                                  bool x_bf16, int kdim, int arow) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wr_row = tid >> 1, wr_half = tid & 1;
  const int xt = tid >> 2, xs = tid & 3;
  const int ar = lane & 31, kh = 8 * (lane >> 5);
  MfmaStage<FMT> st;
  mfma_fetch<FMT>(st, wq, wrow, 32 * wr_half, xrow_ptr ? xrow_ptr + 16 * xs : nullptr, kdim);
#pragma unroll 1
  for (int kc = 0; kc < kdim; kc += 64) {
    __syncthreads();  // the previous chunk's MFMAs are done with the tiles
    mfma_stage_store<FMT>(st, sm, wr_row, wr_half, xt, xs, x_bf16);
    __syncthreads();
    if (kc + 64 < kdim)
      mfma_fetch<FMT>(st, wq, wrow, kc + 64 + 32 * wr_half, xrow_ptr ? xrow_ptr + kc + 64 + 16 * xs : nullptr, kdim);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint16_t* ap = sm.w + arow * TS + 16 * s + kh;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[tt] = mfma32<FMT>(ap, sm.x + (32 * tt + ar) * TS + 16 * s + kh, acc[tt]);
    }
  }
}

// gate/up item: 64 row pairs (n0 ..) x 64 tokens; LDS rows 0..63 gate, 64..127 up.
template <int FMT>
__device__ void mfma_up(const LayerArgs& a, const QMat& G, const QMat& Uq, int mat, const ItemTok& it, int n0,
                        FfnSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  mfma_tables(a, it, sm);
  __syncthreads();
  const int wr_row = tid >> 1;
  QMat wq;
  wq.codes = (wr_row < 64) ? G.codes : Uq.codes;
  wq.scales = (wr_row < 64) ? G.scales : Uq.scales;
  wq.ts = nullptr;
  const size_t wrow = (size_t)mat * D_FF + n0 + (wr_row & 63);
  const int xtok = sm.tok[tid >> 2];
  const uint16_t* xrow = xtok >= 0 ? a.x + (size_t)xtok * D_MODEL : nullptr;
  // A-row r -> LDS row (r < 16 ? 16w + r : 64 + 16w + r - 16): gate and up of the same n
  const int ar = lane & 31;
  const int arow = (ar < 16) ? (16 * wave + ar) : (64 + 16 * wave + ar - 16);
  f32x16 acc[2] = {};
  mfma_kloop<FMT>(acc, sm, wq, wrow, xrow, true, D_MODEL, arow);
  // acc[tt][4i+j] = A-row 8i + 4(lane/32) + j, token 32tt + lane%32:
  // gate for i in {0,1}, the matching up at i+2.
  const float tsg = (FMT == FMT_NVFP4) ? G.ts[mat] : 1.f;
  const float tsu = (FMT == FMT_NVFP4) ? Uq.ts[mat] : 1.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int hrow = sm.row[32 * tt + ar];
    if (hrow < 0) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint16_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = h_store<FMT>(silu_mul(acc[tt][4 * i + j] * tsg, acc[tt][4 * (i + 2) + j] * tsu));
      const int n = n0 + 16 * wave + 8 * i + 4 * (lane >> 5);
      uint2 pk;
      pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
      pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
      *reinterpret_cast<uint2*>(a.h + (size_t)hrow * D_FF + n) = pk;
    }
  }
  __syncthreads();  // tables and tiles are reused by the next item
}

// down item: 128 rows (r0 ..) x 64 tokens, K = 512.
template <int FMT>
__device__ void mfma_down(const LayerArgs& a, const QMat& D, int mat, const ItemTok& it, int r0, FfnSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  mfma_tables(a, it, sm);
  __syncthreads();
  const size_t wrow = (size_t)mat * D_MODEL + r0 + (tid >> 1);
  const int hrow_x = sm.row[tid >> 2];
  const uint16_t* xrow = hrow_x >= 0 ? a.h + (size_t)hrow_x * D_FF : nullptr;
  const int ar = lane & 31;
  f32x16 acc[2] = {};
  mfma_kloop<FMT>(acc, sm, D, wrow, xrow, false, D_FF, 32 * wave + ar);
  const float ts = (FMT == FMT_NVFP4) ? D.ts[mat] : 1.f;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int yrow = sm.row[32 * tt + ar];
    if (yrow < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 32 * wave + 8 * i + 4 * (lane >> 5);
      *reinterpret_cast<float4*>(a.y + (size_t)yrow * D_MODEL + r) =
          make_float4(acc[tt][4 * i] * ts, acc[tt][4 * i + 1] * ts, acc[tt][4 * i + 2] * ts, acc[tt][4 * i + 3] * ts);
    }
  }
  __syncthreads();
}

// ======================================================================================
// Persistent kernels
// ======================================================================================
// Workgroups per CU the persistent kernels are compiled for: two for the 4-bit
// formats (their rings fit in half the register file), one for bf16.
template <int FMT> constexpr int FFN_WG_PER_CU = (FMT == FMT_BF16) ? 1 : 2;

// Items of the matrix-core path come first; the vector-path chunks follow.
template <int FMT, bool SHARED>
__global__ __launch_bounds__(256, FFN_WG_PER_CU<FMT>) void ffn_up_kernel(LayerArgs a) {
  __shared__ union {
    FfnSmem mf;
    GvSmem gv;
  } sm;
  const bool shared_mfma = bucket_mfma(a.T);
  const int n_all = SHARED ? shared_items(a.T, N_UP_CHUNKS) : a.ctl[CTL_N_UP];
  const int n_mf = SHARED ? (shared_mfma ? n_all : 0) : a.ctl[CTL_N_UP_MF];
  for (int i = blockIdx.x; i < n_mf; i += gridDim.x) {
    const Item item = fetch_item<SHARED>(a, a.items_up, i, N_UP_CHUNKS);
    const int e = SHARED ? 0 : item_expert(item.head);
    mfma_up<FMT>(a, SHARED ? a.sh_gate : a.gate, SHARED ? a.sh_up : a.up, e, item_tokens(item, SHARED),
                 item_chunk(item.head) * UP_ROWS, sm.mf);
  }
  if (SHARED) {
    if (!shared_mfma) up_stream<FMT, true>(a, nullptr, n_all, sm.gv);
  } else {
    up_stream<FMT, false>(a, a.items_up + n_mf, n_all - n_mf, sm.gv);
  }
}

template <int FMT, bool SHARED>
__global__ __launch_bounds__(256, FFN_WG_PER_CU<FMT>) void ffn_down_kernel(LayerArgs a) {
  __shared__ union {
    FfnSmem mf;
    GvSmem gv;
  } sm;
  const bool shared_mfma = bucket_mfma(a.T);
  const int n_all = SHARED ? shared_items(a.T, N_DN_CHUNKS) : a.ctl[CTL_N_DN];
  const int n_mf = SHARED ? (shared_mfma ? n_all : 0) : a.ctl[CTL_N_DN_MF];
  for (int i = blockIdx.x; i < n_mf; i += gridDim.x) {
    const Item item = fetch_item<SHARED>(a, a.items_dn, i, N_DN_CHUNKS);
    const int e = SHARED ? 0 : item_expert(item.head);
    const ItemTok it = item_tokens(item, SHARED);
    const int r0 = item_chunk(item.head) * DN_ROWS;
#pragma unroll 1
    for (int rb = 0; rb < DN_ROWS; rb += 128) mfma_down<FMT>(a, SHARED ? a.sh_down : a.down, e, it, r0 + rb, sm.mf);
  }
  if (SHARED) {
    if (!shared_mfma) down_stream<FMT, true>(a, nullptr, n_all, sm.gv);
  } else {
    down_stream<FMT, false>(a, a.items_dn + n_mf, n_all - n_mf, sm.gv);
  }
}

// Workgroups of `kernel` that fit on one CU at once (the persistent kernels are
// launched with exactly the resident count, so none waits for a free slot).
template <typename Kern>
int resident_per_cu(Kern kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

template <int FMT, bool SHARED>
hipError_t launch_ffn_kernel(const LayerArgs& a, bool up, int n_cu, int max_wgs, hipStream_t s) {
  static const int occ_up = resident_per_cu(ffn_up_kernel<FMT, SHARED>);
  static const int occ_dn = resident_per_cu(ffn_down_kernel<FMT, SHARED>);
  int grid = n_cu * (up ? occ_up : occ_dn);
  if (max_wgs < grid) grid = max_wgs;
  if (grid < 1) return hipSuccess;
  if (up) hipLaunchKernelGGL((ffn_up_kernel<FMT, SHARED>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_down_kernel<FMT, SHARED>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_ffn_fmt(const LayerArgs& a, bool up, bool shared, int n_cu, int max_wgs, hipStream_t s) {
  return shared ? launch_ffn_kernel<FMT, true>(a, up, n_cu, max_wgs, s)
                : launch_ffn_kernel<FMT, false>(a, up, n_cu, max_wgs, s);
}

hipError_t launch_ffn(const LayerArgs& a, bool up, bool shared, int n_cu, int max_wgs, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: return launch_ffn_fmt<FMT_Q4_1>(a, up, shared, n_cu, max_wgs, s);
    case FMT_NVFP4: return launch_ffn_fmt<FMT_NVFP4>(a, up, shared, n_cu, max_wgs, s);
    default: return launch_ffn_fmt<FMT_BF16>(a, up, shared, n_cu, max_wgs, s);
  }
}

// ======================================================================================
// Combine and stack glue: one workgroup per token, 8 consecutive columns per thread.
// ======================================================================================
__device__ inline float block_sum256(float v) {
  __shared__ float red[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ inline void store_bf16x8(uint16_t* dst, const float* v) {
  u32x4 pk;
#pragma unroll
  for (int q = 0; q < 4; ++q) pk[q] = (uint32_t)f32_to_bf16(v[2 * q]) | ((uint32_t)f32_to_bf16(v[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4*>(dst) = pk;
}

// xn = bf16(v / sqrt(mean(v^2) + eps)) over the token's 2048 values.
__device__ inline void rmsnorm_store(const float* v, uint16_t* dst, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) ss += v[q] * v[q];
  ss = block_sum256(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D_MODEL + eps);
  float o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = v[q] * inv;
  store_bf16x8(dst, o);
}

// out = sum_j w_j y[slot j] + shared_scale y[shared], in the order j = 0..K-1
// then the shared expert, rounded once to bf16.  Single layer: written to
// a.out.  Stack: recorded to a.y_rec (if any), r += out, then the next
// layer's input bf16(RMSNorm(r)) or, after the last layer, bf16(r).
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) {
  const int t = blockIdx.x;
  const int i0 = 8 * threadIdx.x;
  float o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = 0.f;
  for (int j = 0; j < a.K; ++j) {
    const float wj = a.w[(size_t)t * a.K + j];
    const float4* p = reinterpret_cast<const float4*>(a.y + (size_t)a.inv_perm[(size_t)t * a.K + j] * D_MODEL + i0);
    const float4 v0 = p[0], v1 = p[1];
    o[0] += wj * v0.x; o[1] += wj * v0.y; o[2] += wj * v0.z; o[3] += wj * v0.w;
    o[4] += wj * v1.x; o[5] += wj * v1.y; o[6] += wj * v1.z; o[7] += wj * v1.w;
  }
  if (a.n_shared) {
    const float s = a.shared_scale;
    const float4* p = reinterpret_cast<const float4*>(a.y + (size_t)(a.S + t) * D_MODEL + i0);
    const float4 v0 = p[0], v1 = p[1];
    o[0] += s * v0.x; o[1] += s * v0.y; o[2] += s * v0.z; o[3] += s * v0.w;
    o[4] += s * v1.x; o[5] += s * v1.y; o[6] += s * v1.z; o[7] += s * v1.w;
  }
  if (!a.r) {
    store_bf16x8(a.out + (size_t)t * D_MODEL + i0, o);
    return;
  }
  float yb[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) yb[q] = bf16_to_f32(f32_to_bf16(o[q]));
  if (a.y_rec) store_bf16x8(a.y_rec + (size_t)t * D_MODEL + i0, yb);
  float4* rp = reinterpret_cast<float4*>(a.r + (size_t)t * D_MODEL + i0);
  const float4 r0 = rp[0], r1 = rp[1];
  float rv[8] = {r0.x + yb[0], r0.y + yb[1], r0.z + yb[2], r0.w + yb[3],
                 r1.x + yb[4], r1.y + yb[5], r1.z + yb[6], r1.w + yb[7]};
  rp[0] = make_float4(rv[0], rv[1], rv[2], rv[3]);
  rp[1] = make_float4(rv[4], rv[5], rv[6], rv[7]);
  if (a.x_final) store_bf16x8(a.x_final + (size_t)t * D_MODEL + i0, rv);
  if (a.xn_next) rmsnorm_store(rv, a.xn_next + (size_t)t * D_MODEL + i0, a.eps);
}

hipError_t launch_combine(const LayerArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Stack entry: r = x (fp32), xn = bf16(RMSNorm(r)).
__global__ __launch_bounds__(256) void stack_init_kernel(const uint16_t* __restrict__ x, float* __restrict__ r,
                                                         uint16_t* __restrict__ xn, float eps) {
  const int t = blockIdx.x;
  const int i0 = 8 * threadIdx.x;
  const u32x4 pk = *reinterpret_cast<const u32x4*>(x + (size_t)t * D_MODEL + i0);
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) { v[2 * q] = __uint_as_float(pk[q] << 16); v[2 * q + 1] = __uint_as_float(pk[q] & 0xFFFF0000u); }
  float4* rp = reinterpret_cast<float4*>(r + (size_t)t * D_MODEL + i0);
  rp[0] = make_float4(v[0], v[1], v[2], v[3]);
  rp[1] = make_float4(v[4], v[5], v[6], v[7]);
  rmsnorm_store(v, xn + (size_t)t * D_MODEL + i0, eps);
}

hipError_t launch_stack_init(const uint16_t* x, float* r, uint16_t* xn, int T, float eps, hipStream_t s) {
  hipLaunchKernelGGL(stack_init_kernel, dim3(T), dim3(256), 0, s, x, r, xn, eps);
  return hipGetLastError();
}

}  // namespace moe
