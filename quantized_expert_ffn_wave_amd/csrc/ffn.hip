// Expert FFN over the work lists: gate/up projection with fused SwiGLU, down
// projection, the weighted combine, and the residual/RMSNorm glue of stacked
// layers.
//
// The review "Recursive Flint 40B-A2.5B" (orcarouter.ai), section "The
// architecture is an argument about memory bandwidth", argues that decoding
// this model is a weight-movement problem: each token touches 6 routed experts
// and the shared one out of 257 per layer.  So the work is organised around
// streaming each touched expert's packed weights from HBM once:
//   * buckets below mfma_min(T) tokens (groups of up to 4 tokens) run as a GEMV on
//     v_mfma_f32_4x4x4_16b: a lane loads one 32-element chunk of a weight row
//     (16 bytes of 4-bit codes and the block scale), unpacks it in registers,
//     and the 16 independent 4x4x4 products return it the group's partial sums
//     of its own row; each wave keeps a ring of loads in flight across chunks;
//   * larger buckets (65 tokens on in batches of up to 128 tokens, 16 on in
//     larger ones) run as token tiles of 64 (batches of up to 256 tokens) or
//     128 tokens, so that an expert's weights stream once per tile: each lane
//     loads and decodes its weights straight into the A operand of
//     v_mfma_f32_32x32x16, the tile's activations are staged in LDS, and the
//     next K-chunks are prefetched into registers during the MFMAs.
// Both kernels are persistent and walk device-side work lists that hold the
// routed and the shared expert alike, so no host synchronisation is needed.
//
// Combine: a separate kernel sums, per token, the K weighted expert rows in
// the fixed order j = 0..K-1 and the shared expert row, and rounds once to
// bf16 (in a stack it also updates the fp32 residual and writes the next
// layer's RMSNorm input).
#include <type_traits>

#include "common.hpp"

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte loads: streaming (read once, non-temporal hint) or cached.
template <bool NT> __device__ inline u32x4 ld16(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT> __device__ inline u32x2 ld8(const void* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return *reinterpret_cast<const u32x2*>(p);
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
// operands, so the mask rides in an SGPR and the magic must sit in a VGPR;
// with both as literals the compiler splits this into an AND and an OR.  The
// empty asm hides the constant (it emits no instruction), so it is kept in a
// VGPR and the compiler itself selects v_and_or_b32 and tracks its hazards.
__device__ inline uint32_t magic_vgpr() {
  uint32_t m = MAGIC;
  asm volatile("" : "+v"(m));
  return m;
}
__device__ inline uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic_v) { return (w & mask) | magic_v; }

__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ inline bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// E2M1 pair (byte B of w) -> fp16 pair, unscaled (exact).
template <int B> __device__ inline uint32_t fp4x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B));
}

// two bf16 (lo, hi halves of v) times a power of two sc -> packed fp16 pair.
// Exact wherever the scaled value is an fp16 normal: with sc from pow2_scale
// of the row maximum that is every element above 2^-28 of that maximum (a
// bf16 significand has 8 bits, an fp16 one 11).
__device__ inline uint32_t bf16x2_to_f16x2(uint32_t v, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16) * sc,
                                                                  __uint_as_float(v & 0xFFFF0000u) * sc));
}

// two fp32 values times a power of two sc -> packed fp16 pair, rounded toward zero
__device__ inline uint32_t f32x2_to_f16x2(uint32_t lo, uint32_t hi, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(lo) * sc, __uint_as_float(hi) * sc));
}

// largest |bf16| of the 8 elements in v, as bits (finite inputs)
__device__ inline uint32_t bf16_absmax8(const u32x4& v) {
  uint32_t m = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) m = max(m, max(v[q] & 0x7FFFu, (v[q] >> 16) & 0x7FFFu));
  return m;
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

// Operand precision of the expert GEMMs: fp16 for the 4-bit formats (their
// decoded values are exact in fp16), bf16 for bf16 weights.  The activations
// (x, and the SwiGLU output h, stored as bf16) enter the fp16 products scaled
// per token by a power of two (pow2_scale of the row's largest magnitude),
// which is undone in fp32 on the products' sums: fp16's 5-bit exponent then
// never limits the range of a token row.
template <int FMT> constexpr bool OPER_F16 = FMT != FMT_BF16;
// Element of the stored SwiGLU output h: fp32 where the down product runs on
// scaled fp16 operands (the scale is found from the whole row, after every
// gate/up item has written it), bf16 for bf16 weights.
template <int FMT> using HElem = std::conditional_t<OPER_F16<FMT>, float, uint16_t>;
// Element of the expert outputs y: fp32 for the 4-bit formats, bf16 bits for
// bf16 weights (rounded once, RNE; the combine sums 7 of them in fp32).
template <int FMT> using YElem = std::conditional_t<OPER_F16<FMT>, float, uint16_t>;
template <int FMT> __device__ inline void store_y(const LayerArgs& a, uint32_t off, float v) {
  if constexpr (OPER_F16<FMT>) static_cast<float*>(a.y)[off] = v;
  else static_cast<uint16_t*>(a.y)[off] = f32_to_bf16(v);
}

// ======================================================================================
// Per-format chunk of a weight row: 32 consecutive elements of one row, the
// unit one lane loads (16 bytes of 4-bit codes plus the block scales, or 64
// bytes of bf16), and its decode to fp16/bf16 pairs for the matrix-core tiles.
// ======================================================================================
template <int FMT> struct GV;

// Position of the scales of 32-element block `chunk` within a row of
// cols / 32 blocks: (chunk mod 16) * (cols / 512) + chunk / 16 where 16 divides
// the block count (the natural order for 512 columns).
__device__ inline uint32_t scale_slot(int chunk, int cols) {
  const int C = cols / 32, G = (C % 16 == 0) ? 16 : C;
  return (uint32_t)((chunk % G) * (C / G) + chunk / G);
}
static_assert(D_MODEL / 32 == 64 && D_FF / 32 == 16,
              "the matrix-core loop spells the order out for rows of 64 blocks; rows of 16 keep the natural order");

template <> struct GV<FMT_Q4_1> {
  struct Raw { u32x4 c; uint32_t dm; };                // 16 B codes + fp16 {d, m}
  using Scales4 = u32x4;                               // {d, m} of blocks b, b + 16, b + 32, b + 48
  // chunk `chunk` of row (row + sub); the row terms are workgroup-uniform, the
  // unsigned lane terms let the loads take the scalar-base + vector-offset form
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    return load_slot<NT>(q, row, sub, chunk, scale_slot(chunk, cols), cols);
  }
  // with the block's scale position given (slot = scale_slot(chunk, cols))
  template <bool NT>
  static __device__ Raw load_slot(const QMat& q, size_t row, uint32_t sub, int chunk, uint32_t slot, int cols) {
    Raw r = load_codes<NT>(q, row, sub, chunk, cols);
    r.dm = ld4<NT>(reinterpret_cast<const uint32_t*>(q.scales) + row * (cols / 32) + (sub * (uint32_t)(cols / 32) + slot));
    return r;
  }
  template <bool NT> static __device__ Raw load_codes(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    r.c = ld16<NT>(q.codes + row * (cols / 2) + (sub * (uint32_t)(cols / 2) + 16u * (uint32_t)chunk));
    r.dm = 0u;
    return r;
  }
  // the scales of blocks b + 16 i, i < 4, of a row of 2048 (adjacent in storage)
  template <bool NT> static __device__ Scales4 load_scales4(const QMat& q, size_t row, uint32_t sub, uint32_t b) {
    return ld16<NT>(reinterpret_cast<const uint8_t*>(q.scales) + row * (D_MODEL / 32 * 4) +
                    (sub * (uint32_t)(D_MODEL / 32 * 4) + 16u * b));
  }
  static __device__ void set_scale(Raw& r, const Scales4& s, int i) { r.dm = s[i]; }
  // 32 decoded weights as 16 fp16 pairs in nibble order: fp16(d*q + m), rounded once.
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
  using Scales4 = u32x2;                               // the 2 scales of blocks b, b + 16, b + 32, b + 48
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    return load_slot<NT>(q, row, sub, chunk, scale_slot(chunk, cols), cols);
  }
  template <bool NT>
  static __device__ Raw load_slot(const QMat& q, size_t row, uint32_t sub, int chunk, uint32_t slot, int cols) {
    Raw r = load_codes<NT>(q, row, sub, chunk, cols);
    r.s = ld2<NT>(reinterpret_cast<const uint8_t*>(q.scales) + row * (cols / 16) + (sub * (uint32_t)(cols / 16) + 2u * slot));
    return r;
  }
  template <bool NT> static __device__ Raw load_codes(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    r.c = ld16<NT>(q.codes + row * (cols / 2) + (sub * (uint32_t)(cols / 2) + 16u * (uint32_t)chunk));
    r.s = 0u;
    return r;
  }
  template <bool NT> static __device__ Scales4 load_scales4(const QMat& q, size_t row, uint32_t sub, uint32_t b) {
    return ld8<NT>(reinterpret_cast<const uint8_t*>(q.scales) + row * (D_MODEL / 16) +
                   (sub * (uint32_t)(D_MODEL / 16) + 8u * b));
  }
  static __device__ void set_scale(Raw& r, const Scales4& s, int i) { r.s = (s[i >> 1] >> (16 * (i & 1))) & 0xFFFFu; }
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
  using Scales4 = uint32_t;                            // (no scales)
  template <bool NT>
  static __device__ Raw load_slot(const QMat& q, size_t row, uint32_t sub, int chunk, uint32_t, int cols) {
    return load<NT>(q, row, sub, chunk, cols);
  }
  template <bool NT> static __device__ Scales4 load_scales4(const QMat&, size_t, uint32_t, uint32_t) { return 0u; }
  static __device__ void set_scale(Raw&, const Scales4&, int) {}
  template <bool NT> static __device__ Raw load(const QMat& q, size_t row, uint32_t sub, int chunk, int cols) {
    Raw r;
    const uint8_t* p = q.codes + row * cols * 2 + (sub * (uint32_t)(cols * 2) + 64u * (uint32_t)chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = ld16<NT>(p + 16 * i);
    return r;
  }
  static __device__ void decode(const Raw& r, uint32_t* o) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = r.c[i >> 2][i & 3];
  }
};

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
// Tokens of an item: bucket positions p0 .. p0+cnt-1 of a routed expert
// (expert-output row p: the row of h and of its |h| slots; y is written at the
// position's slot perm[p] instead), or tokens p0 .. p0+cnt-1 of the shared
// expert (row S + t of h and of y).  Vector-path items carry their token ids.
struct ItemTok {
  int p0, cnt;
  bool shared, mfma;
};

__device__ inline ItemTok item_tokens(const Item& item) {
  ItemTok r;
  r.shared = item_shared(item.head);
  r.mfma = item_mfma(item.head);
  r.p0 = (int)item.p0;
  r.cnt = item_count(item.head);
  return r;
}
__device__ inline int row_of(const LayerArgs& a, const ItemTok& it, int i) {
  return it.shared ? a.S + it.p0 + i : it.p0 + i;
}


// ======================================================================================
// Vector-path items
// ======================================================================================

// ======================================================================================
// Vector path (buckets below mfma_min(T) tokens) on the matrix cores.
//
// v_mfma_f32_4x4x4_16b_{f16,bf16} performs 16 independent 4x4x4 products per
// wave: lane l = 4b + j supplies row j of block b's first operand and column j
// of its second one, and receives column j of block b's result.  Here block b
// is one 32-element chunk of the reduction dimension, the first operand holds
// the activations of the item's tokens (up to 4) and the second one 4 weight
// rows.  So lane 4b + j streams chunk b of weight row j -- one 16-byte code
// load plus the block scale, as a plain GEMV lane would -- and gets back the
// 4 tokens' partial sums of its own row: the block scale applies inside the
// lane, and a row's total is the sum over the 16 chunk lanes, taken once per
// 4-row group.  The matrix cores take the token dimension, so the vector ALUs
// only decode weights, whatever the item's token count.
//
// A persistent workgroup walks its chunks c = blockIdx.x, +gridDim.x, ...: a
// chunk is one token group of one expert times VR row pairs (gate/up; UP_ROWS,
// or 16 / 32 in batches of 1 / up to 8 tokens) or VDR rows (down; DN_ROWS, or
// 128 up to 8 tokens), and each wave takes a quarter of the rows.  The chunk's
// activations sit in LDS in operand order (double buffered: the next chunk's
// are loaded during this one), and each wave keeps a ring of weight loads in
// flight that runs on into the next chunk, so the weight stream does not drain
// between chunks.
// ======================================================================================
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int FMT> __device__ inline f32x4 mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
  const u32x2 x = {a0, a1}, w = {b0, b1};
  if constexpr (FMT == FMT_BF16)
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(i16x4, x), __builtin_bit_cast(i16x4, w), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, x), __builtin_bit_cast(f16x4, w), c, 0, 0, 0);
}

template <int FMT> constexpr int MV_UP_RING = (FMT == FMT_BF16) ? 4 : 8;  // weight loads in flight per wave
template <int FMT> constexpr int MV_DN_RING = (FMT == FMT_BF16) ? 4 : 8;
// loads per wave per gate/up item of VR row pairs: VR / 16 row groups x 4 K-quarters x 2 matrices
template <int VR> constexpr int MV_UP_UNITS = VR / 2;
// loads per wave per down item of VDR rows: one per 4-row group (K = 512 in one load)
template <int VDR> constexpr int MV_DN_UNITS = VDR / 16;
// The ring carries loads across items in place: the next item's load i is
// issued into the slot its predecessor load NU - D + i vacates, so D must divide NU.
static_assert(MV_UP_UNITS<16> % MV_UP_RING<FMT_Q4_1> == 0 && MV_UP_UNITS<16> % MV_UP_RING<FMT_BF16> == 0, "ring");
static_assert(MV_DN_UNITS<128> % MV_DN_RING<FMT_Q4_1> == 0 && MV_DN_UNITS<128> % MV_DN_RING<FMT_BF16> == 0, "ring");
constexpr int MV_CHUNKS = D_MODEL / 32;    // 32-element chunks of the longest reduction
constexpr int MV_TOKW = MV_CHUNKS * 16 + 4;  // dwords per token in LDS (16 B of padding against bank conflicts)

// q4_1 per (chunk, token): -1024 * sum(x') seeds the accumulator, S = sum(x)
// weighs the block minimum.
struct MvKS {
  float negK[GV_GROUP];
  float S[GV_GROUP];
};
struct MvSmem {
  uint32_t x[2][GV_GROUP * MV_TOKW];
  MvKS ks[2][MV_CHUNKS];
  float isc[2][GV_GROUP];      // 4-bit formats: inverse activation scale per token
  float hred[2][4][GV_GROUP];  // gate/up, 4-bit formats: each wave's largest |h| per token
};

// token t of a vector-path item, from its packed ids (no indexed array)
__device__ inline int item_token(const Item& item, int t) {
  const uint32_t pair = (t & 2) ? item.t23 : item.t01;
  return (int)((pair >> (16 * (t & 1))) & 0xFFFFu);
}

// One thread per (token, chunk): the chunk's 32 activation elements and, for
// down with the 4-bit formats, two of the row's |h| slots.  The activation
// scale follows at the store: gate/up from the row's largest |x| (a token's 64
// chunks are one wave), down from the largest of the row's 32 |h| slots.
struct MvStage {
  u32x4 v[8];  // 32 bf16 (x, or bf16 h) in v[0..3], or 32 fp32 (h of the 4-bit formats)
  u32x2 hs;    // down, 4-bit formats: the row's |h| slots 2c, 2c + 1
};

template <int FMT, bool UP>
__device__ inline void mv_stage_load(const LayerArgs& a, const Item& item, const ItemTok& it, MvStage& st) {
  constexpr int NCH = UP ? D_MODEL / 32 : D_FF / 32;
  const int t = threadIdx.x / NCH, c = threadIdx.x % NCH;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.v[i] = u32x4{0u, 0u, 0u, 0u};
  st.hs = u32x2{0u, 0u};
  if (t < GV_GROUP && t < it.cnt) {
    const int tok = UP ? item_token(item, t) : 0;
    const int row = UP ? 0 : row_of(a, it, t);
    if constexpr (!UP && OPER_F16<FMT>) {
      const float* src = static_cast<const float*>(a.h) + (size_t)row * D_FF + 32 * c;
#pragma unroll
      for (int i = 0; i < 8; ++i) st.v[i] = ld16<false>(src + 4 * i);
    } else {
      const uint16_t* src = UP ? a.x + (size_t)tok * D_MODEL + 32 * c
                               : static_cast<const uint16_t*>(a.h) + (size_t)row * D_FF + 32 * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.v[i] = ld16<false>(src + 8 * i);
    }
    if constexpr (!UP && OPER_F16<FMT>) st.hs = ld8<false>(a.hslot + (size_t)row * HSLOTS + 2 * c);
  }
}

// Activations into LDS in the operand order of the weights' decode: q4_1 in
// nibble order with the odd elements divided by 16 (exact) to match the
// 16 * q in which the high nibbles arrive; the other formats in natural order.
template <int FMT, bool UP>
__device__ inline void mv_stage_store(const MvStage& st, MvSmem& sm, int buf) {
  constexpr int NCH = UP ? D_MODEL / 32 : D_FF / 32;
  const int t = threadIdx.x / NCH, c = threadIdx.x % NCH;
  if (t >= GV_GROUP) return;
  uint32_t n[16], o[16];
  float sc = 1.f;
  if constexpr (!UP && OPER_F16<FMT>) {  // fp32 h, scaled into fp16 pairs by the row's largest |h|:
    // the maximum over its 32 slots, 2 per thread, reduced over the token's 16 threads (one wave)
    float m = fmaxf(__uint_as_float(st.hs[0]), __uint_as_float(st.hs[1]));
#pragma unroll
    for (int off = 1; off < NCH; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
    sc = pow2_scale(__float_as_uint(m));
#pragma unroll
    for (int i = 0; i < 16; ++i) n[i] = f32x2_to_f16x2(st.v[i >> 1][2 * (i & 1)], st.v[i >> 1][2 * (i & 1) + 1], sc);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) n[4 * i + e] = st.v[i][e];
    }
    if constexpr (OPER_F16<FMT>) {  // bf16 x, scaled into fp16 by its row's largest |x| (the wave's)
      static_assert(!UP || NCH == 64, "a token's chunks fill one wave");
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, bf16_absmax8(st.v[i]));
      sc = pow2_scale(wave_max_u32(m) << 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) n[i] = bf16x2_to_f16x2(n[i], sc);
    }
  }
  if constexpr (OPER_F16<FMT>)
    if (c == 0) sm.isc[buf][t] = pow2_inv(sc);
  if constexpr (FMT == FMT_Q4_1) {
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    float se = 0.f, so = 0.f;  // sums of x' over the even and the odd elements
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      q4_order(n[4 * p], n[4 * p + 1], n[4 * p + 2], n[4 * p + 3], &o[4 * p]);
      o[4 * p + 1] = as_u32(as_f16x2(o[4 * p + 1]) * sixteenth);
      o[4 * p + 3] = as_u32(as_f16x2(o[4 * p + 3]) * sixteenth);
      se += (f16lo(o[4 * p]) + f16hi(o[4 * p])) + (f16lo(o[4 * p + 2]) + f16hi(o[4 * p + 2]));
      so += (f16lo(o[4 * p + 1]) + f16hi(o[4 * p + 1])) + (f16lo(o[4 * p + 3]) + f16hi(o[4 * p + 3]));
    }
    sm.ks[buf][c].negK[t] = -1024.f * (se + so);
    sm.ks[buf][c].S[t] = se + 16.f * so;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = n[i];
  }
  u32x4* dst = reinterpret_cast<u32x4*>(sm.x[buf] + t * MV_TOKW + c * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
}

// The lane's activations for one K-chunk (token j = lane & 3) and, for q4_1,
// the 4 tokens' accumulator seeds and sums of that chunk.
template <int FMT>
__device__ inline void mv_acts(const MvSmem& sm, int buf, int chunk, int j, uint32_t* xq, f32x4& negK, f32x4& S) {
  const u32x4* src = reinterpret_cast<const u32x4*>(sm.x[buf] + j * MV_TOKW + chunk * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = src[i];
    xq[4 * i] = v[0]; xq[4 * i + 1] = v[1]; xq[4 * i + 2] = v[2]; xq[4 * i + 3] = v[3];
  }
  if (FMT == FMT_Q4_1) {
    const MvKS& k = sm.ks[buf][chunk];
    negK = f32x4{k.negK[0], k.negK[1], k.negK[2], k.negK[3]};
    S = f32x4{k.S[0], k.S[1], k.S[2], k.S[3]};
  }
}

// One weight load (32 elements of one row) against the 4 tokens' activations:
// acc[t] += sum_k x_tk w_k.
template <int FMT> struct MV;

template <> struct MV<FMT_Q4_1> {
  // With the nibbles ORed into fp16 1024, the products give
  // sum(x' w') = K + sum(q x), K = 1024 sum(x'); the block dot is
  // d (sum(x' w') - K) + m sum(x).
  static __device__ void unit(const GV<FMT_Q4_1>::Raw& r, const uint32_t* xq, f32x4 negK, f32x4 S, f32x4& acc) {
    const uint32_t mg = magic_vgpr();
    f32x4 d = negK;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w = r.c[p], w8 = w >> 8;
      d = mfma4<FMT_Q4_1>(xq[4 * p], xq[4 * p + 1], and_or(w, 0x000F000Fu, mg), and_or(w, 0x00F000F0u, mg), d);
      d = mfma4<FMT_Q4_1>(xq[4 * p + 2], xq[4 * p + 3], and_or(w8, 0x000F000Fu, mg), and_or(w8, 0x00F000F0u, mg),
                          d);
    }
    const float sc = f16lo(r.dm), mn = f16hi(r.dm);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = fmaf(sc, d[t], fmaf(mn, S[t], acc[t]));
  }
};

template <> struct MV<FMT_NVFP4> {
  // E2M1 * E4M3 is exact in fp16, so the block scales go into the operand and
  // the products accumulate straight on; the per-matrix scale comes after.
  static __device__ void unit(const GV<FMT_NVFP4>::Raw& r, const uint32_t* xq, f32x4, f32x4, f32x4& acc) {
    const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(r.s, 0);
    const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8(r.s, 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f16x2 s = (p < 2) ? f16x2{s0, s0} : f16x2{s1, s1};
      const uint32_t w = r.c[p];
      acc = mfma4<FMT_NVFP4>(xq[4 * p], xq[4 * p + 1], as_u32(as_f16x2(fp4x2_to_f16x2<0>(w)) * s),
                             as_u32(as_f16x2(fp4x2_to_f16x2<1>(w)) * s), acc);
      acc = mfma4<FMT_NVFP4>(xq[4 * p + 2], xq[4 * p + 3], as_u32(as_f16x2(fp4x2_to_f16x2<2>(w)) * s),
                             as_u32(as_f16x2(fp4x2_to_f16x2<3>(w)) * s), acc);
    }
  }
};

template <> struct MV<FMT_BF16> {
  static __device__ void unit(const GV<FMT_BF16>::Raw& r, const uint32_t* xq, f32x4, f32x4, f32x4& acc) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      acc = mfma4<FMT_BF16>(xq[2 * m], xq[2 * m + 1], r.c[m >> 1][2 * (m & 1)], r.c[m >> 1][2 * (m & 1) + 1], acc);
  }
};

// Sum over the 16 chunk lanes (lane bits 2..5) of 8 values per lane, lo[t]
// and hi[t].  Afterwards a lane with bit 2 clear holds, for its row (lane
// bits 0..1), value (bit 5 ? hi : lo)[2 * bit 4 + bit 3].
__device__ inline float mv_reduce8(f32x4 lo, f32x4 hi) {
  const float a0 = halve_step<32>(lo[0], hi[0]), a1 = halve_step<32>(lo[1], hi[1]);
  const float a2 = halve_step<32>(lo[2], hi[2]), a3 = halve_step<32>(lo[3], hi[3]);
  const float b0 = halve_step<16>(a0, a2), b1 = halve_step<16>(a1, a3);
  const float c0 = halve_step<8>(b0, b1);
  // partner lane + 4 inside the row of 16 lanes (DPP row_ror 12)
  return c0 + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(c0), 0x12C, 0xF, 0xF, false));
}

// Weight matrices of a chunk's expert (uniform across the workgroup).
struct ChunkW {
  QMat g, u;   // gate/up (or the down matrix in g)
  int mat;
  float tsg, tsu;
};

// a or b, chosen field by field (a chosen reference would live in scratch)
__device__ inline QMat sel_qmat(bool first, const QMat& x, const QMat& y) {
  QMat q;
  q.codes = first ? x.codes : y.codes;
  q.scales = first ? x.scales : y.scales;
  q.ts = first ? x.ts : y.ts;
  return q;
}

template <int FMT, bool UP>
__device__ inline ChunkW chunk_weights(const LayerArgs& a, const Item& item) {
  ChunkW w;
  const bool sh = item_shared(item.head);
  const int e = sh ? 0 : item_expert(item.head);
  w.mat = e;
  if (UP) {
    w.g = sel_qmat(sh, a.sh_gate, a.gate);
    w.u = sel_qmat(sh, a.sh_up, a.up);
  } else {
    w.g = sel_qmat(sh, a.sh_down, a.down);
    w.u = w.g;
  }
  w.tsg = (FMT == FMT_NVFP4) ? w.g.ts[e] : 1.f;
  w.tsu = (FMT == FMT_NVFP4) ? w.u.ts[e] : 1.f;
  return w;
}

// The item of a chunk is the same for the whole workgroup: keep it in SGPRs so
// that the row addresses derived from it are scalar.
// Item idx of a list with `chunks` row chunks per tile.
__device__ inline Item fetch_item(const Item* tiles, int idx, int chunks) {
  Item it = tiles[idx / chunks];
  it.head |= (uint32_t)(idx % chunks) << 9;
  it.head = __builtin_amdgcn_readfirstlane(it.head);
  it.p0 = __builtin_amdgcn_readfirstlane(it.p0);
  it.t01 = __builtin_amdgcn_readfirstlane(it.t01);
  it.t23 = __builtin_amdgcn_readfirstlane(it.t23);
  return it;
}

// value of lane ^ 32 in the lanes below 32
__device__ inline float upper_half(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}

// Order of the vector-path items c in [0, n) over the G workgroups, given that
// workgroups 0 .. m-1 first took matrix-core items (each worth about two vector
// items at the batch sizes that have both): the first P = R (G - m) items go
// round-robin to the other G - m workgroups only (R rounds), the rest to all
// workgroups round-robin.  With no matrix-core items this is c = blockIdx.x,
// + G, ...
// The walkers are workgroups wid = 0 .. nwg - 1 (the whole grid, or a part of
// a persistent one).
struct VecOrder {
  int G, m, P, w;
  __device__ VecOrder(int n_mf, int wid, int nwg) {
    G = nwg;
    w = wid;
    m = min(n_mf, G);
    const int R = (n_mf > 0 && m < G) ? 2 * ceil_div(n_mf, G) : 0;
    P = R * (G - m);
  }
  __device__ int first() const { return (w >= m && P > 0) ? w - m : P + w; }
  __device__ int next(int c) const {
    if (c < P) {
      const int nc = c + (G - m);
      return nc < P ? nc : P + w;
    }
    return c + G;
  }
};

// The item's largest |h| per token (over its 4 waves' partial maxima in LDS,
// after a barrier) into the |h| slots of the item's VR columns of each token's
// expert-output row.  Items partition a row's columns, so every slot is written
// once per forward and down can take the row's maximum without atomics.
template <int VR>
__device__ inline void vec_hslots(const LayerArgs& a, const Item& item, const ItemTok& it, const MvSmem& sm, int buf) {
  static_assert(VR % 16 == 0, "an item covers whole slots");
  const int t = threadIdx.x;
  if (t < it.cnt) {
    const float m = fmaxf(fmaxf(sm.hred[buf][0][t], sm.hred[buf][1][t]), fmaxf(sm.hred[buf][2][t], sm.hred[buf][3][t]));
    float* dst = a.hslot + (size_t)row_of(a, it, t) * HSLOTS + item_chunk(item.head) * (VR / 16);
#pragma unroll
    for (int i = 0; i < VR / 16; ++i) dst[i] = m;
  }
}

// gate/up + SwiGLU over the vector-path items base + c, c in [0, n), this
// workgroup taking its items in VecOrder.
template <int FMT, int VR>
__device__ void up_stream(const LayerArgs& a, int base, int n, int n_mf, MvSmem& sm, int wid, int nwg) {
  using G = GV<FMT>;
  constexpr int CH = D_FF / VR;
  constexpr int D = MV_UP_RING<FMT>, NU = MV_UP_UNITS<VR>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, b = lane >> 2;
  const VecOrder order(n_mf, wid, nwg);
  int c = order.first();
  if (c >= n) return;
  Item item = fetch_item(a.tiles, base + c, CH);
  ItemTok it = item_tokens(item);
  ChunkW w = chunk_weights<FMT, true>(a, item);
  // load u of a chunk: row group g = u / 8, K-quarter q = (u / 2) % 4, matrix
  // u % 2 (gate, up); lane (b, j) reads chunk 16 q + b of row first_row + 4 g + j
  auto first_row = [&](const Item& itm, const ChunkW& cw) {
    return (size_t)cw.mat * D_FF + item_chunk(itm.head) * VR + wave * (VR / 4);
  };
  // 4-bit formats: the codes ride in the ring, the scales of a row group's 4
  // K-quarters come in one load per matrix (adjacent in storage) and are
  // handed to each unit as it is used
  constexpr bool S4 = FMT != FMT_BF16;
  static_assert(!S4 || D == 8, "scale loads follow the ring's 8-load row groups");
  auto load_unit = [&](const ChunkW& cw, size_t r0, int u) {
    const QMat& q = (u & 1) ? cw.u : cw.g;
    if constexpr (S4) return G::template load_codes<true>(q, r0 + 4 * (u >> 3), (uint32_t)j, 16 * ((u >> 1) & 3) + b, D_MODEL);
    else return G::template load<true>(q, r0 + 4 * (u >> 3), (uint32_t)j, 16 * ((u >> 1) & 3) + b, D_MODEL);
  };
  // the scales of row group u / 8 of load u's matrix
  auto load_sc = [&](const ChunkW& cw, size_t r0, int u) {
    return G::template load_scales4<true>((u & 1) ? cw.u : cw.g, r0 + 4 * (u >> 3), (uint32_t)j, (uint32_t)b);
  };
  size_t r0 = first_row(item, w);
  typename G::Raw ring[D];
  typename G::Scales4 s4c[2] = {}, s4n[2] = {};  // scales of the current / next row group, gate and up
#pragma unroll
  for (int i = 0; i < D; ++i) ring[i] = load_unit(w, r0, i);
  if constexpr (S4) {
    s4c[0] = load_sc(w, r0, 0);
    s4c[1] = load_sc(w, r0, 1);
  }
  int buf = 0;
  {
    MvStage st;
    mv_stage_load<FMT, true>(a, item, it, st);
    mv_stage_store<FMT, true>(st, sm, buf);
  }
  __syncthreads();
  // after each group's reduction, lanes with bits 5 and 2 clear hold gate
  // sums of token 2 * bit 4 + bit 3 (the matching up sums sit in lane + 32)
  const int my_t = ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
#pragma unroll 1
  for (;;) {
    const int nc = order.next(c);
    const bool has_next = nc < n;
    Item nitem = item;
    ItemTok nit = it;
    ChunkW nw = w;
    size_t nr0 = r0;
    MvStage st;
    if (has_next) {
      nitem = fetch_item(a.tiles, base + nc, CH);
      nit = item_tokens(nitem);
      nw = chunk_weights<FMT, true>(a, nitem);
      nr0 = first_row(nitem, nw);
      mv_stage_load<FMT, true>(a, nitem, nit, st);
    }
    const bool writer = (lane & 36) == 0 && my_t < it.cnt;
    const int hrow = row_of(a, it, 0) + my_t;
    // the lane's h elements, as a 32-bit offset from the uniform base (one VGPR, not a 64-bit pointer)
    const uint32_t hoff = (uint32_t)(hrow * D_FF + item_chunk(item.head) * VR + wave * (VR / 4) + j);
    const float isc = OPER_F16<FMT> ? sm.isc[buf][my_t] : 1.f;  // undoes the token's activation scale
    float hm = 0.f;                                             // largest |h| this lane writes
    f32x4 acc[2] = {}, negK = {}, S = {};
    uint32_t xq[16];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int g = u >> 3, q = (u >> 1) & 3, m = u & 1;
      if (m == 0) {
        mv_acts<FMT>(sm, buf, 16 * q + b, j, xq, negK, S);
        if (q == 0) acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      typename G::Raw cur = ring[u % D];
      if constexpr (S4) G::set_scale(cur, s4c[m], q);
      const int un = u + D;  // the load issued now
      if (un < NU) {
        ring[u % D] = load_unit(w, r0, un);
        if (S4 && ((un >> 1) & 3) == 0) s4n[m] = load_sc(w, r0, un);
      } else if (has_next) {
        ring[u % D] = load_unit(nw, nr0, un - NU);
        if (S4 && (((un - NU) >> 1) & 3) == 0) s4n[m] = load_sc(nw, nr0, un - NU);
      }
      MV<FMT>::unit(cur, xq, negK, S, acc[m]);
      if (u % 8 == 7) {
        if constexpr (S4) {
          s4c[0] = s4n[0];
          s4c[1] = s4n[1];
        }
        float v = mv_reduce8(acc[0], acc[1]);
        if (FMT == FMT_NVFP4) v *= (lane & 32) ? w.tsu : w.tsg;
        if constexpr (OPER_F16<FMT>) v *= isc;
        const float up = upper_half(v);
        const float hv = silu_mul(v, up);
        if (writer) {
          if constexpr (OPER_F16<FMT>) static_cast<float*>(a.h)[hoff + 4 * g] = hv;
          else static_cast<uint16_t*>(a.h)[hoff + 4 * g] = f32_to_bf16(hv);
          hm = fmaxf(hm, fabsf(hv));
        }
      }
    }
    if constexpr (OPER_F16<FMT>) {  // the wave's largest |h| per token (a quad holds 4 rows of one token)
      hm = fmaxf(hm, dpp_partner<1>(hm));
      hm = fmaxf(hm, dpp_partner<2>(hm));
      if ((lane & 39) == 0) sm.hred[buf][wave][my_t] = hm;  // lanes 0, 8, 16, 24: tokens 0..3
    }
    if (!has_next) break;
    mv_stage_store<FMT, true>(st, sm, buf ^ 1);
    __syncthreads();
    if constexpr (OPER_F16<FMT>) vec_hslots<VR>(a, item, it, sm, buf);
    buf ^= 1;
    c = nc;
    item = nitem;
    it = nit;
    w = nw;
    r0 = nr0;
  }
  if constexpr (OPER_F16<FMT>) {
    __syncthreads();
    vec_hslots<VR>(a, item, it, sm, buf);
  }
}

// down over vector-path chunks, ordered and loaded as in up_stream: load u of a
// chunk covers rows first_row + 4 u + j over the whole K = 512 (chunk b per lane)
template <int FMT, int VDR>
__device__ void down_stream(const LayerArgs& a, int base, int n, int n_mf, MvSmem& sm, int wid, int nwg) {
  using G = GV<FMT>;
  constexpr int CH = D_MODEL / VDR;
  constexpr int D = MV_DN_RING<FMT>, NU = MV_DN_UNITS<VDR>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, b = lane >> 2;
  const VecOrder order(n_mf, wid, nwg);
  int c = order.first();
  if (c >= n) return;
  Item item = fetch_item(a.tiles, base + c, CH);
  ItemTok it = item_tokens(item);
  ChunkW w = chunk_weights<FMT, false>(a, item);
  auto first_row = [&](const Item& itm, const ChunkW& cw) {
    return (size_t)cw.mat * D_MODEL + item_chunk(itm.head) * VDR + wave * (VDR / 4);
  };
  auto load_unit = [&](const ChunkW& cw, size_t r0, int u) {
    return G::template load<true>(cw.g, r0 + 4 * u, (uint32_t)j, b, D_FF);
  };
  size_t r0 = first_row(item, w);
  typename G::Raw ring[D];
#pragma unroll
  for (int i = 0; i < D; ++i) ring[i] = load_unit(w, r0, i);
  int buf = 0;
  {
    MvStage st;
    mv_stage_load<FMT, false>(a, item, it, st);
    mv_stage_store<FMT, false>(st, sm, buf);
  }
  __syncthreads();
  // after a reduction over two row groups, lanes with bit 2 clear hold row
  // group (2 p + bit 5)'s sum for token 2 * bit 4 + bit 3
  const int my_t = ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
  // the lane's y row: token my_t's slot (from perm), or S + token (shared);
  // the next item's is read just before the ring's first load of that item,
  // so that waiting for it waits for no load of the next item
  auto y_row = [&](const ItemTok& x) {
    return x.shared ? a.S + x.p0 + my_t : a.perm[x.p0 + min(my_t, x.cnt - 1)];
  };
  int yrow = y_row(it);
#pragma unroll 1
  for (;;) {
    const int nc = order.next(c);
    const bool has_next = nc < n;
    Item nitem = item;
    ItemTok nit = it;
    ChunkW nw = w;
    size_t nr0 = r0;
    int nyrow = yrow;
    MvStage st;
    if (has_next) {
      nitem = fetch_item(a.tiles, base + nc, CH);
      nit = item_tokens(nitem);
      nw = chunk_weights<FMT, false>(a, nitem);
      nr0 = first_row(nitem, nw);
      mv_stage_load<FMT, false>(a, nitem, nit, st);
    }
    const bool writer = (lane & 4) == 0 && my_t < it.cnt;
    const float isc = OPER_F16<FMT> ? sm.isc[buf][my_t] : 1.f;  // undoes the row's h scale
    // the lane's y elements, as a 32-bit offset from the uniform base
    const uint32_t yoff = (uint32_t)(yrow * D_MODEL + item_chunk(item.head) * VDR +
                                     wave * (VDR / 4) + 4 * ((lane >> 5) & 1) + j);
    uint32_t xq[16];
    f32x4 negK = {}, S = {};
    mv_acts<FMT>(sm, buf, b, j, xq, negK, S);
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const typename G::Raw cur = ring[u % D];
      if (u + D < NU) {
        ring[u % D] = load_unit(w, r0, u + D);
      } else if (has_next) {
        if (u + D == NU) nyrow = y_row(nit);
        ring[u % D] = load_unit(nw, nr0, u + D - NU);
      }
      acc[u & 1] = f32x4{0.f, 0.f, 0.f, 0.f};
      MV<FMT>::unit(cur, xq, negK, S, acc[u & 1]);
      if (u & 1) {
        float v = mv_reduce8(acc[0], acc[1]);
        if (FMT == FMT_NVFP4) v *= w.tsg;
        if constexpr (OPER_F16<FMT>) v *= isc;
        if (writer) store_y<FMT>(a, yoff + 4 * (u - 1), v);
      }
    }
    if (!has_next) break;
    mv_stage_store<FMT, false>(st, sm, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    c = nc;
    item = nitem;
    it = nit;
    w = nw;
    r0 = nr0;
    yrow = nyrow;
  }
}

// ======================================================================================
// Matrix-core items.  Each wave owns RB blocks of 32 weight rows and loads them
// straight from global memory into the A operand of v_mfma_f32_32x32x16_{f16,bf16}:
// lane (r = lane % 32, h = lane / 32) holds, for each 64-wide K-chunk and row
// block, the 32 weights k = 32 h .. 32 h + 31 of its row (one block of the 4-bit
// formats), decoded into the chunk's 4 MFMA steps of 8 weights.  The chunk's
// BN-token activation tile is staged in LDS (double buffered, one barrier per
// chunk) in the decode's k order, and lane (token c = lane % 32, h) reads the
// same k of its token as the B operand.  NS K-chunks are held in registers: the
// one multiplied and the NS - 1 loads in flight behind it.
//   gate/up item (4 waves x 32 RB row pairs from n0): with RB = 2 a wave's block
//     0 holds gate rows n0 + 32 w + r and block 1 the up rows of the same n; with
//     RB = 1 its one block holds gate rows n0 + 16 w + r (r < 16) and the up rows
//     of the same n (r >= 16).  Either way a lane holds both inputs of its SwiGLU
//     outputs.  RB = 2 for 128-token tiles (fewer passes over the activation
//     tile when the batch is large), 1 for 64-token ones (more, shorter items);
//   down item: DN_ROWS rows from r0; wave w's block b = rows r0 + 64 w + 32 b + r.
// ======================================================================================
constexpr int TS = 72;  // LDS row stride in 16-bit elements (64 + 8 pad)
template <int BN> constexpr int MF_TT = BN / 32;         // 32-token blocks of a tile
template <int BN> constexpr int MF_XT = 256 / BN;        // threads per token when staging activations
template <int BN> constexpr int MF_XK = 64 / MF_XT<BN>;  // activation elements per thread and K-chunk
template <int BN> constexpr int MF_UP_RB = (BN == 128) ? 2 : 1;
// K-chunks held in registers: gate/up (K = 2048) 4, or 2 where 4 would not fit
// two waves per SIMD (128-token tiles); down (K = 512, 8 chunks) 2
template <int FMT, int BN> constexpr int MF_NS_UP = (BN == 128) ? 2 : 4;
template <int FMT, int BN> constexpr int MF_NS_DN = 2;
static_assert(MF_XK<64> % 16 == 0 && MF_XK<128> % 16 == 0, "activations are staged 16 elements at a time");
static_assert(DN_ROWS == 4 * 64, "down items: 4 waves x 2 row blocks of 32 rows");
static_assert(D_MODEL % (64 * 4) == 0 && D_FF % (64 * 4) == 0, "the chunk loop is unrolled by up to 4");

// Weights reach the matrix cores through LDS (mf_kloop_bf16, mf_kloop_q): a
// block of 64 rows x 128 bytes per wave (one K-chunk of bf16, four of the 4-bit
// codes), single-buffered: only its own wave uses it.
template <int FMT> constexpr int MF_WL_ROWS = 64;
// Down items, 4-bit formats: the block scales of each wave's 64 rows, one row
// (D_FF / 32 blocks: 64 bytes q4_1, 32 NVFP4) per DN_SW words, padded by a word
// so that the 32 lanes reading one word of 32 rows hit 32 banks.
template <int FMT> constexpr int DN_SW = (FMT == FMT_Q4_1) ? D_FF / 32 + 1 : (FMT == FMT_NVFP4) ? D_FF / 64 + 1 : 1;
// (64-token tiles only: the 128-token tiles keep the per-lane loop, and their LDS two workgroups per CU)
template <int FMT, int BN> constexpr int DN_SWORDS = (FMT != FMT_BF16 && BN == 64) ? 64 * DN_SW<FMT> : 1;
template <int FMT, int BN> struct FfnSmem {
  uint16_t x[2][BN * TS];  // K-chunks alternate between the two, so one barrier per chunk suffices
  uint16_t w[4][MF_WL_ROWS<FMT> * TS];  // bf16 weights: each wave's rows of the current K-chunk
  int tok[BN];
  int row[BN];             // h rows (bucket positions; shared: S + token)
  int yrow[BN];            // y rows (slots t K + j; shared: S + token)
  float sc[BN];            // 4-bit formats: activation scale per token column (down: from |h|)
  float isc[BN];           // and its inverse
  float hred[4][BN];       // gate/up, 4-bit formats: each wave's largest |h| per token column
  uint32_t ds[4][DN_SWORDS<FMT, BN>];  // down, 4-bit formats: each wave's block scales
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
__device__ inline f32x16 mfma32(u32x4 av, u32x4 bv, f32x16 c) {
  if (OPER_F16<FMT>)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, bv), c, 0,
                                                  0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0,
                                                 0, 0);
}

// UP: the activation scale is the token's (x); down: the expert-output row's
// (h), from the maximum over the row's 32 |h| slots, read by 256 / BN threads
// per token column and reduced over them.
template <int FMT, bool UP, int BN>
__device__ inline void mfma_tables(const LayerArgs& a, const ItemTok& it, FfnSmem<FMT, BN>& sm) {
  const int i = threadIdx.x;
  if (i < BN) {
    // matrix-core tiles are shared-expert tiles or routed buckets (tokens via perm)
    const int slot = (i < it.cnt && !it.shared) ? a.perm[it.p0 + i] : 0;
    const int tok = (i < it.cnt) ? (it.shared ? it.p0 + i : slot / a.K) : -1;
    const int row = (i < it.cnt) ? row_of(a, it, i) : -1;
    sm.tok[i] = tok;
    sm.row[i] = row;
    sm.yrow[i] = (i < it.cnt) ? (it.shared ? row : slot) : -1;
    if (UP && OPER_F16<FMT>) {
      const float sc = (i < it.cnt) ? a.xsc[tok] : 1.f;
      sm.sc[i] = sc;
      sm.isc[i] = pow2_inv(sc);
    }
  }
  if constexpr (!UP && OPER_F16<FMT>) {
    constexpr int P = 256 / BN, NS = HSLOTS / P;  // threads per token column, slots per thread
    static_assert(P == 2 || P == 4, "2 or 4 threads per column: one DPP exchange each");
    const int col = i / P, part = i % P;
    float m = 0.f;
    if (col < it.cnt) {
      const u32x4* src = reinterpret_cast<const u32x4*>(a.hslot + (size_t)row_of(a, it, col) * HSLOTS + NS * part);
#pragma unroll
      for (int k = 0; k < NS / 4; ++k) {
        const u32x4 v = src[k];
        m = fmaxf(fmaxf(m, fmaxf(__uint_as_float(v[0]), __uint_as_float(v[1]))),
                  fmaxf(__uint_as_float(v[2]), __uint_as_float(v[3])));
      }
    }
    m = fmaxf(m, dpp_partner<1>(m));
    if (P == 4) m = fmaxf(m, dpp_partner<2>(m));
    if (part == 0) {
      const float sc = pow2_scale(__float_as_uint(m));
      sm.sc[col] = sc;
      sm.isc[col] = pow2_inv(sc);
    }
  }
}

// One K-chunk in registers: the lane's 32 weights of each row block, and the
// thread's MF_XK activations of token tid / MF_XT (elements MF_XK * (tid % MF_XT) ..).
template <int FMT, int BN, int RB, bool XF32> struct MfStage {
  typename GV<FMT>::Raw w[RB];
  u32x4 x[MF_XK<BN> / (XF32 ? 4 : 8)];  // the thread's activations: bf16, or fp32 (h of the 4-bit formats)
};

// acc[b][tt] += W_block_b (this wave's rows) x X (tokens 32 tt ..) over K = kdim.
// q[b], wrow[b]: the matrix and the lane's weight row of block b; xsrc: the
// thread's activation row (bf16, or fp32 with XF32) and offset (a valid row
// also for tokens past the tile's count: their columns are never stored, and a
// column only meets its own activations); xscale: that row's activation scale
// (4-bit formats).
template <int FMT, int BN, int RB, int NS, bool XF32 = false>
__device__ inline void mf_kloop(f32x16 (&acc)[RB][MF_TT<BN>], FfnSmem<FMT, BN>& sm, const QMat (&q)[RB],
                                const size_t (&wrow)[RB], const void* xsrc, float xscale, int kdim) {
  using Stage = MfStage<FMT, BN, RB, XF32>;
  constexpr int NX = MF_XK<BN> / (XF32 ? 4 : 8);  // 16-byte activation loads per thread and chunk
  static_assert(!XF32 || OPER_F16<FMT>, "fp32 activations feed the fp16 products only");
  static_assert(NS % 2 == 0, "chunk j uses LDS buffer j % 2");
  const int tid = threadIdx.x, lane = tid & 63;
  const int h = lane >> 5, c = lane & 31;
  const int xt = tid / MF_XT<BN>, xs = tid % MF_XT<BN>;
  const int nc = kdim / 64;
  // every load is issued unconditionally (past the last chunk the last one is
  // loaded again), so that the compiler's wait counts stay exact
  auto fetch = [&](Stage& st, int ck) {
    ck = min(ck, nc - 1);
    // scale position of block 2 ck + h: with 2048 columns the blocks are stored
    // in the order k mod 16, k / 16, i.e. at 8 (ck mod 8) + 4 h + ck / 8
    const uint32_t slot = (kdim == D_MODEL) ? 8u * (uint32_t)(ck & 7) + 4u * (uint32_t)h + (uint32_t)(ck >> 3)
                                            : 2u * (uint32_t)ck + (uint32_t)h;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if constexpr (FMT == FMT_NVFP4 && BN == 64) {
        // the aligned 4 bytes holding the slot's 2, shifted into place at the
        // decode: a 16-bit load result is narrowed and widened again at the
        // top of the loop, and that wait drains every load in flight (not for
        // 128-token tiles, whose registers are full)
        st.w[b] = GV<FMT>::template load_codes<false>(q[b], wrow[b], 0u, 2 * ck + h, kdim);
        st.w[b].s = ld4<false>(static_cast<const uint8_t*>(q[b].scales) + wrow[b] * (kdim / 16) + 4 * (slot >> 1));
      } else {
        st.w[b] = GV<FMT>::template load_slot<false>(q[b], wrow[b], 0u, 2 * ck + h, slot, kdim);
      }
    }
#pragma unroll
    for (int i = 0; i < NX; ++i)
      st.x[i] = ld16<false>(static_cast<const uint8_t*>(xsrc) + (XF32 ? 4 : 2) * 64 * ck + 16 * i);
  };
  auto stage = [&](const Stage& st, uint16_t* buf) {
#pragma unroll
    for (int g = 0; g < MF_XK<BN> / 16; ++g) {
      uint32_t xv[8];
      if constexpr (XF32) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          xv[i] = f32x2_to_f16x2(st.x[4 * g + i / 2][2 * (i & 1)], st.x[4 * g + i / 2][2 * (i & 1) + 1], xscale);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = st.x[2 * g + i / 4][i % 4];
        if constexpr (OPER_F16<FMT>) {
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = bf16x2_to_f16x2(xv[i], xscale);
        }
      }
      stage_x16<FMT>(buf + xt * TS + MF_XK<BN> * xs + 16 * g, xv);
    }
  };
  auto multiply = [&](const Stage& st, int ck, const uint16_t* buf) {
    uint32_t wv[RB][16];
    // NVFP4: which half of the scale dword is the lane's (slot mod 2, as in fetch)
    const int shift = 16 * ((kdim == D_MODEL) ? ((ck >> 3) & 1) : h);
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      typename GV<FMT>::Raw r = st.w[b];
      if constexpr (FMT == FMT_NVFP4 && BN == 64) r.s >>= shift;
      GV<FMT>::decode(r, wv[b]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s);
#pragma unroll
        for (int b = 0; b < RB; ++b)
          acc[b][tt] = mfma32<FMT>(u32x4{wv[b][4 * s], wv[b][4 * s + 1], wv[b][4 * s + 2], wv[b][4 * s + 3]}, bv,
                                   acc[b][tt]);
      }
    }
  };
  Stage st[NS];
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) fetch(st[i], i);
#pragma unroll 1
  for (int ck0 = 0; ck0 < nc; ck0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      // Keep each chunk's work in its place: left free, the scheduler hoists the
      // weight decodes of all NS chunks to the top of the unrolled body, and
      // their wait drains every load in flight (the prefetch then buys nothing).
      __builtin_amdgcn_sched_barrier(0);
      stage(st[j], sm.x[j & 1]);
      fetch(st[(j + NS - 1) % NS], ck0 + j + NS - 1);
      __syncthreads();
      multiply(st[j], ck0 + j, sm.x[j & 1]);
    }
  }
}

// bf16 weights: acc[b][tt] += W_block_b x X over K = kdim with both operands
// staged in LDS.  Every global load is line-friendly: a lane loads 16 bytes and 8
// lanes cover one 128-byte piece (64 K-elements) of a row, so one load
// instruction reads 8 whole cache lines: 8 of the wave's 32 RB weight rows, or 8
// of the tile's tokens.  (Loading each lane's own MFMA operand instead touches
// 32 rows per instruction, which streams from HBM at half the rate.)  The
// weights are regrouped into the A layout through the wave's LDS block, the
// activations through the shared tile as in mf_kloop; chunk j's global loads are
// issued NS - 1 chunks ahead.  xbase + xrow[t] * kdim: the bf16 row of tile
// token t (xrow in LDS, rows past cnt repeat a valid one; their columns are
// never stored).  The wave's 32 RB weight rows are two halves of 16 RB
// consecutive rows each, starting at rows wh[0] and wh[1] (gate and up rows of
// the same outputs, or two blocks of down rows); wave row r sits in LDS row r,
// so block b of the A operand is LDS rows 32 b ..
template <int BN, int RB, int NS>
__device__ inline void mf_kloop_bf16(f32x16 (&acc)[RB][MF_TT<BN>], FfnSmem<FMT_BF16, BN>& sm,
                                     const uint16_t* const (&wh)[2], const uint16_t* xbase, const int* xrow, int cnt,
                                     int kdim) {
  constexpr int NW = 4 * RB;   // weight loads per lane and chunk: wave rows 8 i + lane / 8
  constexpr int HR = 16 * RB;  // rows per half
  constexpr int NX = BN / 32;  // activation loads per thread and chunk: tokens 32 i + 8 wave + lane / 8
  static_assert(NS % 2 == 0, "chunk j uses activation buffer j % 2");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31, sub = lane >> 3, part = lane & 7;
  const int nc = kdim / 64;
  uint16_t* wl = sm.w[wave];
  const uint16_t* wp[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) wp[g] = wh[g] + (size_t)sub * kdim + 8 * part;
  uint32_t xo[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) xo[i] = (uint32_t)xrow[min(32 * i + 8 * wave + sub, cnt - 1)] * (uint32_t)kdim + 8u * part;
  struct Stage {
    u32x4 w[NW];
    u32x4 x[NX];
  };
  auto fetch = [&](Stage& st, int ck) {
    ck = min(ck, nc - 1);  // past the last chunk the last one is loaded again (exact wait counts)
#pragma unroll
    for (int i = 0; i < NW; ++i)
      st.w[i] = ld16<true>(wp[(8 * i) / HR] + (size_t)((8 * i) % HR) * kdim + 64 * ck);
#pragma unroll
    for (int i = 0; i < NX; ++i) st.x[i] = ld16<false>(xbase + xo[i] + 64 * ck);
  };
  auto stage = [&](const Stage& st, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4*>(wl + (8 * i + sub) * TS + 8 * part) = st.w[i];
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(buf + (32 * i + 8 * wave + sub) * TS + 8 * part) = st.x[i];
  };
  auto multiply = [&](const uint16_t* buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 av[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) av[b] = *reinterpret_cast<const u32x4*>(wl + (32 * b + c) * TS + 32 * h + 8 * s);
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s);
#pragma unroll
        for (int b = 0; b < RB; ++b) acc[b][tt] = mfma32<FMT_BF16>(av[b], bv, acc[b][tt]);
      }
    }
  };
  Stage st[NS];
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) fetch(st[i], i);
#pragma unroll 1
  for (int ck0 = 0; ck0 < nc; ck0 += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      stage(st[j], sm.x[j & 1]);
      fetch(st[(j + NS - 1) % NS], ck0 + j + NS - 1);
      __syncthreads();
      multiply(sm.x[j & 1]);
    }
  }
}

// 4-bit weights, gate/up: the same scheme as mf_kloop_bf16 for the codes and
// the activations.  The activations come pre-scaled in fp16 and in the weights'
// k order (xq), so they are copied as they are.  The codes move in groups of
// four K-chunks (128 bytes of a row, one line-friendly load per 8 rows and
// lane), each group staged into the wave's LDS block while the next one is
// loaded; a lane then reads its 16 bytes of a chunk from there and decodes them
// as mf_kloop does.  The block scales: q4_1 loaded per lane, 3 chunks ahead;
// NVFP4 (a row's scales for all of K are one 128-byte line) staged once per
// item into the unused upper half of the wave's LDS block, with line-friendly
// loads like the codes, and read from there per chunk.  (Per-lane scale loads
// touch 32 rows per instruction; on the 256-token NVFP4 layer they cost about
// as much as the whole decode.)
// q[b], wrow[b]: the lane's matrix and row of block b (for its scales); sh: the
// scale rows of the two halves (NVFP4).
template <int FMT, int BN, int RB, int NSX>
__device__ inline void mf_kloop_q(f32x16 (&acc)[RB][MF_TT<BN>], FfnSmem<FMT, BN>& sm, const QMat (&q)[RB],
                                  const size_t (&wrow)[RB], const uint8_t* const (&wh)[2],
                                  const uint8_t* const (&sh)[2], const uint16_t* xbase, const int* xrow, int cnt) {
  constexpr int kdim = D_MODEL;
  constexpr int RBYTES = kdim / 2;  // codes per row
  constexpr int NW = 4 * RB;        // code loads per lane and group: wave rows 8 i + lane / 8
  constexpr int HR = 16 * RB;       // rows per half
  constexpr int NX = BN / 32;       // activation loads per thread and chunk
  constexpr int NC = kdim / 64, NG = NC / 4;
  static_assert(NSX == 4, "activation ring of 4 chunks, as deep as the scales'");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31, sub = lane >> 3, part = lane & 7;
  uint8_t* wl = reinterpret_cast<uint8_t*>(sm.w[wave]);
  constexpr int WS = TS * 2;  // LDS bytes per weight row
  constexpr bool SL = FMT == FMT_NVFP4;  // scales through LDS
  constexpr int SBYTES = kdim / 16;      // NVFP4 scale bytes per row
  static_assert(!SL || (RB == 1 && 2 * 32 * WS <= MF_WL_ROWS<FMT> * TS * 2 && SBYTES == 128),
                "NVFP4: 32 rows of codes and 32 rows of 128 scale bytes in the wave's LDS block");
  const uint8_t* wp[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) wp[g] = wh[g] + (size_t)sub * RBYTES + 16 * part;
  uint32_t xo[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) xo[i] = (uint32_t)xrow[min(32 * i + 8 * wave + sub, cnt - 1)] * (uint32_t)kdim + 8u * part;
  u32x4 wst[NW];
  u32x4 xst[NSX][NX];
  uint32_t sst[4][RB] = {};  // (q4_1)
  auto fetch_w = [&](int g) {
    g = min(g, NG - 1);
#pragma unroll
    for (int i = 0; i < NW; ++i) wst[i] = ld16<true>(wp[(8 * i) / HR] + (size_t)((8 * i) % HR) * RBYTES + 128 * g);
  };
  auto stage_w = [&]() {
#pragma unroll
    for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4*>(wl + (8 * i + sub) * WS + 16 * part) = wst[i];
  };
  auto fetch_x = [&](u32x4 (&st)[NX], int ck) {
    ck = min(ck, NC - 1);
#pragma unroll
    for (int i = 0; i < NX; ++i) st[i] = ld16<false>(xbase + xo[i] + 64 * ck);
  };
  auto stage_x = [&](const u32x4 (&st)[NX], uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(buf + (32 * i + 8 * wave + sub) * TS + 8 * part) = st[i];
  };
  auto fetch_s = [&](uint32_t (&st)[RB], int ck) {
    ck = min(ck, NC - 1);
    // block 2 ck + h of a row of 2048: stored at 8 (ck mod 8) + 4 h + ck / 8
    const uint32_t slot = 8u * (uint32_t)(ck & 7) + 4u * (uint32_t)h + (uint32_t)(ck >> 3);
#pragma unroll
    for (int b = 0; b < RB; ++b)
      st[b] = ld4<false>(reinterpret_cast<const uint32_t*>(q[b].scales) + wrow[b] * (kdim / 32) + slot);
  };
  auto multiply = [&](int ck, const uint32_t (&sc)[RB], const uint16_t* buf) {
    const int cg = ck & 3;
    uint32_t wv[RB][16];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      typename GV<FMT>::Raw r;
      r.c = *reinterpret_cast<const u32x4*>(wl + (32 * b + c) * WS + 32 * cg + 16 * h);
      if constexpr (FMT == FMT_Q4_1) {
        r.dm = sc[b];
      } else {
        // the aligned 4 bytes holding slot 8 (ck mod 8) + 4 h + ck / 8 (2 bytes
        // each), from the lane's scale row
        const uint32_t w4 = 4u * (uint32_t)(ck & 7) + 2u * (uint32_t)h + (uint32_t)(ck >> 4);
        r.s = *reinterpret_cast<const uint32_t*>(wl + (32 + c) * WS + 4 * w4) >> (16 * ((ck >> 3) & 1));
      }
      GV<FMT>::decode(r, wv[b]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s);
#pragma unroll
        for (int b = 0; b < RB; ++b)
          acc[b][tt] = mfma32<FMT>(u32x4{wv[b][4 * s], wv[b][4 * s + 1], wv[b][4 * s + 2], wv[b][4 * s + 3]}, bv,
                                   acc[b][tt]);
      }
    }
  };
  if constexpr (SL) {
    // wave rows 8 i + lane / 8 of the two halves, 16 bytes per lane; written
    // once the codes and activations of the first chunks are on their way
    u32x4 sl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sl[i] = ld16<false>(sh[(8 * i) / 16] + (size_t)((8 * i) % 16 + sub) * SBYTES + 16 * part);
    fetch_w(0);
#pragma unroll
    for (int i = 0; i < 3; ++i) fetch_x(xst[i], i);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(wl + (32 + 8 * i + sub) * WS + 16 * part) = sl[i];
  } else {
    // the prologue issues its loads in the loop's order (activations, then
    // scales, chunk by chunk): the wait counts at the loop top hold for both
    // ways in, so they stay those of the steady state
    fetch_w(0);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      fetch_x(xst[i], i);
      fetch_s(sst[i], i);
    }
  }
#pragma unroll 1
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ck = 4 * g + j;
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0) {
        stage_w();      // the previous group's chunks are multiplied (this wave, in order)
        fetch_w(g + 1);
      }
      stage_x(xst[j % NSX], sm.x[j & 1]);
      fetch_x(xst[(j + NSX - 1) % NSX], ck + NSX - 1);
      if constexpr (!SL) fetch_s(sst[(j + 3) % 4], ck + 3);
      __syncthreads();
      multiply(ck, sst[j], sm.x[j & 1]);
    }
  }
}

// 4-bit weights, down (K = D_FF: 8 K-chunks, two groups of four), tables
// included.  The codes move as in mf_kloop_q: line-friendly loads of a group
// of four K-chunks staged through the wave's LDS block.  The block scales of
// the wave's 64 rows are contiguous in storage; they are read once per item
// with contiguous loads and kept in LDS (the per-lane loads they replace touch
// 32 rows per instruction, as did the per-lane code loads).  The tables (the
// down half of mfma_tables: rows, and each row's activation scale from its |h|
// slots) read the slots first, then the first group of codes and the scales
// are requested, so that the tables' wait is for the slots alone and the
// codes' latency overlaps it.  The activations (h,
// fp32) are read line-friendly too: 16 threads take a token's 256 bytes of a
// chunk (4 floats each), 16 tokens per round, and convert and store them as
// mf_kloop does (q4_1: the two halves of each 8-element group trade a pair of
// values between neighbouring lanes to reach the weights' k order), 2 chunks
// ahead.  Same products in the same order as mf_kloop with fp32 activations.
template <int FMT, int BN>
__device__ inline void mf_down_q(const LayerArgs& a, const QMat& D, int mat, const ItemTok& it, int r0,
                                 FfnSmem<FMT, BN>& sm, f32x16 (&acc)[2][MF_TT<BN>]) {
  static_assert(FMT != FMT_BF16 && BN == 64, "4-bit formats, 64-token tiles");
  constexpr int kdim = D_FF, RBYTES = kdim / 2, NC = kdim / 64, NG = NC / 4;
  constexpr int SB = (FMT == FMT_Q4_1) ? kdim / 32 * 4 : kdim / 16;  // scale bytes per row
  constexpr int SW = DN_SW<FMT>;
  constexpr int NSL = 64 * SB / 1024;  // 16-byte scale loads per lane
  constexpr int NXR = BN / 16;         // activation loads per thread and chunk
  constexpr int NSX = 3;               // activation chunks in registers
  constexpr int WS = TS * 2;           // LDS bytes per weight row
  static_assert(NG == 2 && 64 * SB % 1024 == 0 && SW * 4 == SB + 4, "rows of 512: two groups, whole scale rows");
  static_assert(MF_WL_ROWS<FMT> == 64, "the wave's 64 code rows of a group fill its LDS block");
  static_assert(DN_SWORDS<FMT, BN> == 64 * SW, "scale rows of the wave's 64 rows");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31, sub = lane >> 3, part = lane & 7;
  uint8_t* wl = reinterpret_cast<uint8_t*>(sm.w[wave]);
  uint32_t* sl = sm.ds[wave];
  const size_t w0 = (size_t)mat * D_MODEL + r0 + 64 * wave;  // the wave's first row
  const uint8_t* wp = D.codes + (w0 + sub) * RBYTES + 16 * part;
  u32x4 wst[8];
  auto fetch_w = [&](int g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wst[i] = ld16<true>(wp + (size_t)(8 * i) * RBYTES + 128 * g);
  };
  auto stage_w = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(wl + (8 * i + sub) * WS + 16 * part) = wst[i];
  };
  // |h| slots of column tid / P (P threads per column; past the count a valid
  // row, ignored), then the codes and scales
  constexpr int P = 256 / BN, NSH = HSLOTS / P;
  static_assert(P == 4 && NSH % 4 == 0, "4 threads per token column: two DPP exchanges");
  const int col = tid / P, pt = tid % P;
  const int yslot = (tid < it.cnt && !it.shared) ? a.perm[it.p0 + tid] : 0;  // y row of token column tid
  u32x4 hv[NSH / 4];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.hslot + (size_t)row_of(a, it, min(col, it.cnt - 1)) * HSLOTS +
                                                      NSH * pt);
#pragma unroll
    for (int k = 0; k < NSH / 4; ++k) hv[k] = src[k];
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4 sst[NSL];
#pragma unroll
  for (int i = 0; i < NSL; ++i)
    sst[i] = ld16<false>(static_cast<const uint8_t*>(D.scales) + w0 * SB + 1024 * i + 16 * lane);
  fetch_w(0);
  __builtin_amdgcn_sched_barrier(0);
  {
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < NSH / 4; ++k)
      m = fmaxf(fmaxf(m, fmaxf(__uint_as_float(hv[k][0]), __uint_as_float(hv[k][1]))),
                fmaxf(__uint_as_float(hv[k][2]), __uint_as_float(hv[k][3])));
    if (col >= it.cnt) m = 0.f;
    m = fmaxf(m, dpp_partner<1>(m));
    m = fmaxf(m, dpp_partner<2>(m));
    if (pt == 0) {
      const float sc = pow2_scale(__float_as_uint(m));
      sm.sc[col] = sc;
      sm.isc[col] = pow2_inv(sc);
    }
    if (tid < BN) {
      sm.row[tid] = (tid < it.cnt) ? row_of(a, it, tid) : -1;
      sm.yrow[tid] = (tid < it.cnt) ? (it.shared ? row_of(a, it, tid) : yslot) : -1;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NSL; ++i) {
    const int o = 1024 * i + 16 * lane;  // byte of the wave's scales
#pragma unroll
    for (int d = 0; d < 4; ++d) sl[(o / SB) * SW + (o % SB) / 4 + d] = sst[i][d];
  }
  // thread: 4 floats (elements 4 q ..) of tokens 16 i + tid / 16 of each chunk
  const int q = tid & 15;
  uint32_t xo[NXR];
  float xs[NXR];
#pragma unroll
  for (int i = 0; i < NXR; ++i) {
    const int t = min(16 * i + (tid >> 4), it.cnt - 1);  // past the count: a valid row, never stored
    xo[i] = (uint32_t)sm.row[t] * (uint32_t)kdim + 4u * (uint32_t)q;
    xs[i] = sm.sc[t];
  }
  const float* hb = static_cast<const float*>(a.h);
  u32x4 xst[NSX][NXR];
  auto fetch_x = [&](u32x4 (&st)[NXR], int ck) {
#pragma unroll
    for (int i = 0; i < NXR; ++i) st[i] = ld16<false>(hb + xo[i] + 64 * ck);
  };
  auto stage_x = [&](const u32x4 (&st)[NXR], uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < NXR; ++i) {
      uint32_t p0 = f32x2_to_f16x2(st[i][0], st[i][1], xs[i]);
      uint32_t p1 = f32x2_to_f16x2(st[i][2], st[i][3], xs[i]);
      if constexpr (FMT == FMT_Q4_1) {
        // even q holds elements 0-3 of an 8-group, odd q 4-7; order 0 4 1 5 | 2 6 3 7
        const bool even = (q & 1) == 0;
        const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)(even ? p1 : p0), 0xB1, 0xF, 0xF, false);
        const uint32_t lo = even ? p0 : got, hi = even ? got : p1;
        p0 = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        p1 = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
      }
      *reinterpret_cast<u32x2*>(buf + (16 * i + (tid >> 4)) * TS + 4 * q) = u32x2{p0, p1};
    }
  };
  auto multiply = [&](int ck, const uint16_t* buf) {
    const int cg = ck & 3;
    uint32_t wv[2][16];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      typename GV<FMT>::Raw r;
      r.c = *reinterpret_cast<const u32x4*>(wl + (32 * b + c) * WS + 32 * cg + 16 * h);
      // block 2 ck + h of the row: q4_1 word 2 ck + h; NVFP4 half h of word ck
      if constexpr (FMT == FMT_Q4_1) r.dm = sl[(32 * b + c) * SW + 2 * ck + h];
      else r.s = sl[(32 * b + c) * SW + ck] >> (16 * h);
      GV<FMT>::decode(r, wv[b]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[b][tt] = mfma32<FMT>(u32x4{wv[b][4 * s], wv[b][4 * s + 1], wv[b][4 * s + 2], wv[b][4 * s + 3]}, bv,
                                   acc[b][tt]);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NSX - 1; ++i) fetch_x(xst[i], i);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ck = 4 * g + j;
      __builtin_amdgcn_sched_barrier(0);
      if (j == 0) {
        stage_w();  // the previous group's chunks are multiplied (this wave, in order)
        if (g + 1 < NG) fetch_w(g + 1);
      }
      stage_x(xst[ck % NSX], sm.x[ck & 1]);
      if (ck + NSX - 1 < NC) fetch_x(xst[(ck + NSX - 1) % NSX], ck + NSX - 1);
      __syncthreads();
      multiply(ck, sm.x[ck & 1]);
    }
  }
}

// gate/up item: 32 MF_UP_RB row pairs per wave (n0 ..) x BN tokens.
template <int FMT, int BN>
__device__ void mfma_up(const LayerArgs& a, const QMat& G, const QMat& Uq, int mat, const ItemTok& it, int n0,
                        FfnSmem<FMT, BN>& sm) {
  constexpr int RB = MF_UP_RB<BN>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  mfma_tables<FMT, true>(a, it, sm);
  __syncthreads();
  QMat q[RB];
  size_t wrow[RB];
  if constexpr (RB == 2) {
    q[0] = G;
    q[1] = Uq;
    wrow[0] = wrow[1] = (size_t)mat * D_FF + n0 + 32 * wave + c;
  } else {
    q[0] = sel_qmat(c < 16, G, Uq);
    wrow[0] = (size_t)mat * D_FF + n0 + 16 * wave + (c & 15);
  }
  const int xtok = sm.tok[min(tid / MF_XT<BN>, it.cnt - 1)];
  const uint16_t* xsrc = a.x + (size_t)xtok * D_MODEL + MF_XK<BN> * (tid % MF_XT<BN>);
  const float xscale = OPER_F16<FMT> ? a.xsc[xtok] : 1.f;
  f32x16 acc[RB][MF_TT<BN>] = {};
  if constexpr (FMT == FMT_BF16) {
    // the wave's gate rows and up rows of the same outputs
    const size_t r = (size_t)mat * D_FF + n0 + 16 * RB * wave;
    const uint16_t* const wh[2] = {reinterpret_cast<const uint16_t*>(G.codes) + r * D_MODEL,
                                   reinterpret_cast<const uint16_t*>(Uq.codes) + r * D_MODEL};
    mf_kloop_bf16<BN, RB, MF_NS_UP<FMT, BN>>(acc, sm, wh, a.x, sm.tok, it.cnt, D_MODEL);
  } else if constexpr (BN == 64) {
    const size_t r = (size_t)mat * D_FF + n0 + 16 * RB * wave;
    const uint8_t* const wh[2] = {G.codes + r * (D_MODEL / 2), Uq.codes + r * (D_MODEL / 2)};
    const uint8_t* const sh[2] = {static_cast<const uint8_t*>(G.scales) + r * (D_MODEL / 16),
                                  static_cast<const uint8_t*>(Uq.scales) + r * (D_MODEL / 16)};
    mf_kloop_q<FMT, BN, RB, 4>(acc, sm, q, wrow, wh, sh, a.xq, sm.tok, it.cnt);
  } else {
    // (128-token tiles: the staged loop's registers do not fit two waves per SIMD)
    mf_kloop<FMT, BN, RB, MF_NS_UP<FMT, BN>>(acc, sm, q, wrow, xsrc, xscale, D_MODEL);
  }
  // acc[b][tt][4i+j] = row 8i + 4h + j of block b, token 32tt + c.  The gate
  // value of a lane's output (block 0 / rows below 16) sits at gi, its up at ui.
  const float tsg = (FMT == FMT_NVFP4) ? G.ts[mat] : 1.f;
  const float tsu = (FMT == FMT_NVFP4) ? Uq.ts[mat] : 1.f;
  constexpr int NI = (RB == 2) ? 4 : 2;  // groups of 4 outputs per lane and token block
#pragma unroll
  for (int tt = 0; tt < MF_TT<BN>; ++tt) {
    const int hrow = sm.row[32 * tt + c];
    // the token's inverse activation scale folds into the tensor scales
    const float isc = OPER_F16<FMT> ? sm.isc[32 * tt + c] : 1.f;
    const float sg = tsg * isc, su = tsu * isc;
    float hm = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float hf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float g = (RB == 2) ? acc[0][tt][4 * i + j] : acc[0][tt][4 * i + j];
        const float u = (RB == 2) ? acc[RB - 1][tt][4 * i + j] : acc[0][tt][4 * (i + 2) + j];
        hf[j] = silu_mul(g * sg, u * su);
        hm = fmaxf(hm, fabsf(hf[j]));
      }
      const int n = n0 + 32 * RB / 2 * wave + 8 * i + 4 * h;
      if (hrow >= 0) {
        if constexpr (OPER_F16<FMT>) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.h) + (size_t)hrow * D_FF + n) =
              make_float4(hf[0], hf[1], hf[2], hf[3]);
        } else {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(hf[0]) | ((uint32_t)f32_to_bf16(hf[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(hf[2]) | ((uint32_t)f32_to_bf16(hf[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h) + (size_t)hrow * D_FF + n) = pk;
        }
      }
    }
    if constexpr (OPER_F16<FMT>) {  // the wave's largest |h| per token column, both lane halves
      hm = fmaxf(hm, upper_half(hm));
      if (h == 0) sm.hred[wave][32 * tt + c] = hm;
    }
  }
  __syncthreads();  // tables and tiles are reused by the next item
  if constexpr (OPER_F16<FMT>) {
    // the item's largest |h| per token into the |h| slots of its D_FF / UC
    // columns (items partition a row's columns: every slot once per forward)
    constexpr int NSL = D_FF / mf_up_chunks(BN) / 16;  // slots of the item's columns
    static_assert(NSL == 4 * RB, "4 waves x 16 RB row pairs");
    const int i = threadIdx.x;
    if (i < it.cnt) {
      const float m = fmaxf(fmaxf(sm.hred[0][i], sm.hred[1][i]), fmaxf(sm.hred[2][i], sm.hred[3][i]));
      float* dst = a.hslot + (size_t)sm.row[i] * HSLOTS + n0 / 16;
#pragma unroll
      for (int k = 0; k < NSL / 4; ++k) *reinterpret_cast<float4*>(dst + 4 * k) = make_float4(m, m, m, m);
    }
    __syncthreads();  // the LDS is taken over by the next item (or the vector path)
  }
}

// down item: DN_ROWS rows (r0 ..) x BN tokens, K = 512.
template <int FMT, int BN>
__device__ void mfma_down(const LayerArgs& a, const QMat& D, int mat, const ItemTok& it, int r0,
                          FfnSmem<FMT, BN>& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31;
  f32x16 acc[2][MF_TT<BN>] = {};
  if constexpr (FMT != FMT_BF16 && BN == 64) {
    mf_down_q<FMT, BN>(a, D, mat, it, r0, sm, acc);
  } else {
    mfma_tables<FMT, false>(a, it, sm);
    __syncthreads();
    const QMat q[2] = {D, D};
    const size_t wr = (size_t)mat * D_MODEL + r0 + 64 * wave + c;
    const size_t wrow[2] = {wr, wr + 32};
    if constexpr (FMT == FMT_BF16) {
      const uint16_t* w0 = reinterpret_cast<const uint16_t*>(D.codes) + (wr - (size_t)c) * D_FF;
      const uint16_t* const wh[2] = {w0, w0 + (size_t)32 * D_FF};
      mf_kloop_bf16<BN, 2, MF_NS_DN<FMT, BN>>(acc, sm, wh, static_cast<const uint16_t*>(a.h), sm.row, it.cnt, D_FF);
    } else {
      const int hrow_x = sm.row[min(tid / MF_XT<BN>, it.cnt - 1)];
      const HElem<FMT>* xsrc =
          static_cast<const HElem<FMT>*>(a.h) + (size_t)hrow_x * D_FF + MF_XK<BN> * (tid % MF_XT<BN>);
      const float xscale = sm.sc[min(tid / MF_XT<BN>, it.cnt - 1)];
      mf_kloop<FMT, BN, 2, MF_NS_DN<FMT, BN>, OPER_F16<FMT>>(acc, sm, q, wrow, xsrc, xscale, D_FF);
    }
  }
  const float tsd = (FMT == FMT_NVFP4) ? D.ts[mat] : 1.f;
#pragma unroll
  for (int tt = 0; tt < MF_TT<BN>; ++tt) {
    const int yrow = sm.yrow[32 * tt + c];
    if (yrow < 0) continue;
    const float ts = OPER_F16<FMT> ? tsd * sm.isc[32 * tt + c] : tsd;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 64 * wave + 32 * b + 8 * i + 4 * h;
        const size_t off = (size_t)yrow * D_MODEL + r;
        if constexpr (OPER_F16<FMT>) {
          *reinterpret_cast<float4*>(static_cast<float*>(a.y) + off) =
              make_float4(acc[b][tt][4 * i] * ts, acc[b][tt][4 * i + 1] * ts, acc[b][tt][4 * i + 2] * ts,
                          acc[b][tt][4 * i + 3] * ts);
        } else {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(acc[b][tt][4 * i] * ts) | ((uint32_t)f32_to_bf16(acc[b][tt][4 * i + 1] * ts) << 16);
          pk.y = (uint32_t)f32_to_bf16(acc[b][tt][4 * i + 2] * ts) | ((uint32_t)f32_to_bf16(acc[b][tt][4 * i + 3] * ts) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + off) = pk;
        }
      }
    }
  }
  __syncthreads();
}

// bf16 down items, one workgroup's sequence idx = i0, i0 + stride, ... < n, as
// one K-loop: the chunk after an item's last one is the next item's first, so
// its loads are in flight during the last chunk's products and the y stores
// instead of after them (an item has only 8 K-chunks, and the first one's
// latency, paid once per item, was about a tenth of it).  No tables: an item's
// h rows are its bucket positions (routed) or S + its tokens (shared),
// contiguous, and its y rows are read from perm with the item.  Same loads, LDS layout and products in the
// same order as mfma_down through mf_kloop_bf16.
__device__ inline int mf_item(int i, int n, int C);
template <int BN>
__device__ void mfma_down_bf16_seq(const LayerArgs& a, int i0, int stride, int n, FfnSmem<FMT_BF16, BN>& sm) {
  constexpr int NW = 8;               // weight loads per lane and chunk: wave rows 8 i + lane / 8
  constexpr int NX = BN / 32;         // h loads per thread and chunk: tokens 32 i + 8 wave + lane / 8
  constexpr int kdim = D_FF, NC = kdim / 64;
  static_assert(MF_NS_DN<FMT_BF16, BN> == 2 && NC % 2 == 0, "two stages, chunk j in LDS buffer j % 2");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31, sub = lane >> 3, part = lane & 7;
  uint16_t* wl = sm.w[wave];
  const uint16_t* hb = static_cast<const uint16_t*>(a.h);
  struct Src {
    const uint16_t* wp;  // the lane's first weight row piece of the wave's 64 rows
    uint32_t xo[NX];     // the thread's h row offsets (elements)
    int yr[MF_TT<BN>];   // the lane's y rows (token columns 32 tt + c; -1 past the count)
    int mat, r0;
  };
  // item idx of the sequence is entry mf_item(idx) of the list (row chunk mf_item(idx) % N_DN_CHUNKS)
  auto prep = [&](const Item& raw, int idx) {
    Item item = raw;
    item.head |= (uint32_t)(mf_item(idx, n, N_DN_CHUNKS) % N_DN_CHUNKS) << 9;
    item.head = __builtin_amdgcn_readfirstlane(item.head);
    item.p0 = __builtin_amdgcn_readfirstlane(item.p0);
    const ItemTok it = item_tokens(item);
    Src s;
    s.mat = it.shared ? 0 : item_expert(item.head);
    s.r0 = item_chunk(item.head) * DN_ROWS;
#pragma unroll
    for (int tt = 0; tt < MF_TT<BN>; ++tt) {
      const int col = 32 * tt + c;
      s.yr[tt] = col >= it.cnt ? -1 : it.shared ? a.S + it.p0 + col : a.perm[it.p0 + col];
    }
    const uint16_t* codes = reinterpret_cast<const uint16_t*>(it.shared ? a.sh_down.codes : a.down.codes);
    s.wp = codes + ((size_t)s.mat * D_MODEL + s.r0 + 64 * wave + sub) * kdim + 8 * part;
#pragma unroll
    for (int i = 0; i < NX; ++i) s.xo[i] = (uint32_t)row_of(a, it, min(32 * i + 8 * wave + sub, it.cnt - 1)) * kdim + 8u * part;
    return s;
  };
  auto load_item = [&](int idx) { return a.tiles[mf_item(idx, n, N_DN_CHUNKS) / N_DN_CHUNKS]; };
  struct Stage {
    u32x4 w[NW];
    u32x4 x[NX];
  };
  auto fetch = [&](Stage& st, const Src& s, int ck) {
#pragma unroll
    for (int i = 0; i < NW; ++i) st.w[i] = ld16<true>(s.wp + (size_t)(8 * i) * kdim + 64 * ck);
#pragma unroll
    for (int i = 0; i < NX; ++i) st.x[i] = ld16<false>(hb + s.xo[i] + 64 * ck);
  };
  auto stage = [&](const Stage& st, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < NW; ++i) *reinterpret_cast<u32x4*>(wl + (8 * i + sub) * TS + 8 * part) = st.w[i];
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(buf + (32 * i + 8 * wave + sub) * TS + 8 * part) = st.x[i];
  };
  f32x16 acc[2][MF_TT<BN>];
  auto multiply = [&](const uint16_t* buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 av[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) av[b] = *reinterpret_cast<const u32x4*>(wl + (32 * b + c) * TS + 32 * h + 8 * s);
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s);
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b][tt] = mfma32<FMT_BF16>(av[b], bv, acc[b][tt]);
      }
    }
  };
  int idx = i0;
  if (idx >= n) return;
  Src cur = prep(load_item(idx), idx);
  Stage st[2];
  fetch(st[0], cur, 0);
  for (;;) {
    const int nidx = idx + stride;
    const bool more = nidx < n;
    // the next item's entry, read now and used at the last chunk
    const Item nraw = load_item(more ? nidx : idx);
#pragma unroll
    for (int tt = 0; tt < MF_TT<BN>; ++tt) acc[0][tt] = acc[1][tt] = f32x16{};
    Src nxt = cur;
#pragma unroll 1
    for (int ck0 = 0; ck0 < NC; ck0 += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ck = ck0 + j;
        __builtin_amdgcn_sched_barrier(0);
        stage(st[j], sm.x[j]);
        if (ck + 1 < NC) {
          fetch(st[j ^ 1], cur, ck + 1);
        } else {
          // past the sequence's last item its last chunk is loaded again (exact wait counts)
          if (more) nxt = prep(nraw, nidx);
          fetch(st[j ^ 1], nxt, more ? 0 : NC - 1);
        }
        __syncthreads();
        multiply(sm.x[j]);
      }
    }
    // y: acc[b][tt][4 i + j] = output row 64 wave + 32 b + 8 i + 4 h + j, token column 32 tt + c
#pragma unroll
    for (int tt = 0; tt < MF_TT<BN>; ++tt) {
      if (cur.yr[tt] < 0) continue;
      const size_t yrow = (size_t)cur.yr[tt];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = cur.r0 + 64 * wave + 32 * b + 8 * i + 4 * h;
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(acc[b][tt][4 * i]) | ((uint32_t)f32_to_bf16(acc[b][tt][4 * i + 1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(acc[b][tt][4 * i + 2]) | ((uint32_t)f32_to_bf16(acc[b][tt][4 * i + 3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y) + yrow * D_MODEL + r) = pk;
        }
      }
    }
    if (!more) break;
    idx = nidx;
    cur = nxt;
  }
  __syncthreads();  // the LDS is taken over by the vector path
}

// bf16 gate/up items of 128-token tiles, one workgroup's sequence idx = i0,
// i0 + stride, ... < n, as one K-loop (as mfma_down_bf16_seq): the next item's
// entry is read when an item starts, its token ids (from perm) halfway through
// its chunks, and its first chunk is loaded during the last chunk's products and
// the SwiGLU stores, instead of a table round trip and a pipeline fill per item.
// No LDS tables: the h rows of an item's token columns are its bucket positions
// (or S + token).  Same loads, LDS layout and products in the same order as
// mfma_up through mf_kloop_bf16.
template <int BN>
__device__ void mfma_up_bf16_seq(const LayerArgs& a, int i0, int stride, int n, FfnSmem<FMT_BF16, BN>& sm) {
  static_assert(BN == 128 && MF_UP_RB<BN> == 2 && MF_NS_UP<FMT_BF16, BN> == 2, "2 row blocks, 2 stages");
  constexpr int UC = mf_up_chunks(BN);  // items per tile (128 row pairs each)
  constexpr int NX = BN / 32;           // x loads per thread and chunk: tokens 32 i + 8 wave + lane / 8
  constexpr int kdim = D_MODEL, NC = kdim / 64;
  static_assert(NC % 2 == 0, "chunk j in LDS buffer j % 2");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, c = lane & 31, sub = lane >> 3, part = lane & 7;
  uint16_t* wl = sm.w[wave];
  struct Cur {
    int p0, cnt, shared, n0;
    size_t wrow;  // the wave's first gate (and up) row in its matrix
  };
  auto decode_item = [&](const Item& raw, int idx) {
    const int m = mf_item(idx, n, UC);
    Cur r;
    const uint32_t head = __builtin_amdgcn_readfirstlane(raw.head);
    r.p0 = (int)__builtin_amdgcn_readfirstlane(raw.p0);
    r.cnt = item_count(head);
    r.shared = item_shared(head);
    r.n0 = (m % UC) * (D_FF / UC);
    r.wrow = (size_t)(r.shared ? 0 : item_expert(head)) * D_FF + r.n0 + 32 * wave;
    return r;
  };
  auto load_item = [&](int idx) { return a.tiles[mf_item(idx, n, UC) / UC]; };
  // the thread's token of x load i, clamped into the item's count
  auto tok_slot = [&](const Cur& r, int i) { return min(32 * i + 8 * wave + sub, r.cnt - 1); };
  struct Stage {
    u32x4 w[8];
    u32x4 x[NX];
  };
  auto fetch = [&](Stage& st, const Cur& r, const uint32_t (&xo)[NX], int ck) {
    const uint16_t* wg = reinterpret_cast<const uint16_t*>(r.shared ? a.sh_gate.codes : a.gate.codes);
    const uint16_t* wu = reinterpret_cast<const uint16_t*>(r.shared ? a.sh_up.codes : a.up.codes);
    const size_t off = (r.wrow + sub) * kdim + 8 * part + 64 * ck;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.w[i] = ld16<true>(wg + off + (size_t)(8 * i) * kdim);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.w[4 + i] = ld16<true>(wu + off + (size_t)(8 * i) * kdim);
#pragma unroll
    for (int i = 0; i < NX; ++i) st.x[i] = ld16<false>(a.x + xo[i] + 64 * ck);
  };
  auto stage = [&](const Stage& st, uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(wl + (8 * i + sub) * TS + 8 * part) = st.w[i];
#pragma unroll
    for (int i = 0; i < NX; ++i) *reinterpret_cast<u32x4*>(buf + (32 * i + 8 * wave + sub) * TS + 8 * part) = st.x[i];
  };
  f32x16 acc[2][MF_TT<BN>];
  auto multiply = [&](const uint16_t* buf) {
#pragma unroll
    for (int s_ = 0; s_ < 4; ++s_) {
      u32x4 av[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) av[b] = *reinterpret_cast<const u32x4*>(wl + (32 * b + c) * TS + 32 * h + 8 * s_);
#pragma unroll
      for (int tt = 0; tt < MF_TT<BN>; ++tt) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (32 * tt + c) * TS + 32 * h + 8 * s_);
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b][tt] = mfma32<FMT_BF16>(av[b], bv, acc[b][tt]);
      }
    }
  };
  int idx = i0;
  if (idx >= n) return;
  Cur cur = decode_item(load_item(idx), idx);
  uint32_t xo[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int j = tok_slot(cur, i);
    xo[i] = (uint32_t)(cur.shared ? cur.p0 + j : a.perm[cur.p0 + j] / a.K) * (uint32_t)kdim + 8u * part;
  }
  Stage st[2];
  fetch(st[0], cur, xo, 0);
  for (;;) {
    const int nidx = idx + stride;
    const bool more = nidx < n;
    const Item nraw = load_item(more ? nidx : idx);  // used halfway through
    Cur nxt = cur;
    int pv[NX];
#pragma unroll
    for (int tt = 0; tt < MF_TT<BN>; ++tt) acc[0][tt] = acc[1][tt] = f32x16{};
#pragma unroll 1
    for (int ck0 = 0; ck0 < NC; ck0 += 2) {
      if (ck0 == NC / 2) {
        // the next item's tokens, read half an item ahead of their use
        nxt = more ? decode_item(nraw, nidx) : cur;
#pragma unroll
        for (int i = 0; i < NX; ++i) pv[i] = nxt.shared ? 0 : a.perm[nxt.p0 + tok_slot(nxt, i)];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ck = ck0 + j;
        __builtin_amdgcn_sched_barrier(0);
        stage(st[j], sm.x[j]);
        if (ck + 1 < NC) {
          fetch(st[j ^ 1], cur, xo, ck + 1);
        } else {
          // past the sequence's last item its last chunk is loaded again (exact wait counts)
          if (more) {
#pragma unroll
            for (int i = 0; i < NX; ++i)
              xo[i] = (uint32_t)(nxt.shared ? nxt.p0 + tok_slot(nxt, i) : pv[i] / a.K) * (uint32_t)kdim + 8u * part;
          }
          fetch(st[j ^ 1], more ? nxt : cur, xo, more ? 0 : NC - 1);
        }
        __syncthreads();
        multiply(sm.x[j]);
      }
    }
    // SwiGLU: acc[b][tt][4 i + j] = row pair n0 + 32 wave + 8 i + 4 h + j (b = 0 gate, 1 up), token column 32 tt + c
#pragma unroll
    for (int tt = 0; tt < MF_TT<BN>; ++tt) {
      const int col = 32 * tt + c;
      if (col >= cur.cnt) continue;
      const size_t hrow = (size_t)(cur.shared ? a.S + cur.p0 + col : cur.p0 + col);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float hf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hf[e] = silu_mul(acc[0][tt][4 * i + e], acc[1][tt][4 * i + e]);
        const int nn = cur.n0 + 32 * wave + 8 * i + 4 * h;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(hf[0]) | ((uint32_t)f32_to_bf16(hf[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(hf[2]) | ((uint32_t)f32_to_bf16(hf[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h) + hrow * D_FF + nn) = pk;
      }
    }
    if (!more) break;
    idx = nidx;
    cur = nxt;
  }
  __syncthreads();  // the LDS is taken over by the vector path
}

// ======================================================================================
// Persistent kernels
// ======================================================================================
// Workgroups per CU the persistent kernels are compiled for: three for the
// vector-only kernels (BN = 0: the ring fits in a third of the register file,
// and a third workgroup keeps more of the weight stream in flight), two where
// matrix-core tiles are possible.  They are launched with as many workgroups
// as are resident at once, at most MF_WG_PER_CU per CU where tiles are possible.
template <int FMT, int BN> constexpr int FFN_WG_PER_CU = (BN == 0 && FMT != FMT_BF16) ? 3 : 2;
constexpr int MF_WG_PER_CU = 2;

// LDS of the persistent kernels: the matrix-core tiles (BN tokens wide) only
// where the batch can have them (BN > 0: T >= mfma_min(T)), since their double
// buffer would otherwise cost the vector path occupancy.
template <int FMT, int BN> struct FfnKernelSmem {
  union {
    FfnSmem<FMT, BN> mf;
    MvSmem gv;
  };
};
template <int FMT> struct FfnKernelSmem<FMT, 0> {
  MvSmem gv;
};

// Matrix-core items in an XCD-aware order.  Workgroups are dispatched to the 8
// XCDs round-robin by blockIdx, and workgroup c takes items c, c + gridDim.x,
// ... (gridDim.x a multiple of 8), so item i runs on XCD i % 8.  In groups of 8
// tiles of C items, position i = 8 C g + 8 ch + tl holds item ch of tile 8 g + tl:
// the items of a tile run on one XCD at about the same time and read its
// activation tile through that XCD's L2 instead of once per XCD.
__device__ inline int mf_item(int i, int n, int C) {
  const int G = 8 * C;
  if (i >= (n / G) * G) return i;
  const int g = i / G, r = i % G, ch = r >> 3, tl = r & 7;
  return (8 * g + tl) * C + ch;
}

// Workgroups that take down items of the matrix-core path: with more items
// than workgroups, the fewest that keep the same number of rounds (a multiple
// of 8, so that item i still runs on XCD i % 8), so that the last round does
// not run half empty.  At 4096 tokens the 2304 down items take 464 of 512
// workgroups for 5 rounds (down 175 -> 172 us).  Not for gate/up: its 1152
// items on 384 workgroups took 268 against 239 us on 512, since an item's
// length is set by its K-loop's latency, not by its share of HBM.
__device__ inline int mf_grid(int n, int g) {
  if (n <= g) return g;
  const int rounds = ceil_div(n, g);
  return min(g, (ceil_div(n, rounds) + 7) & ~7);
}

// Items of the matrix-core path come first; the vector-path chunks follow.
// VR, VDR: rows of the vector-path gate/up and down items (vec_up_rows and
// vec_dn_rows of the batch size).
static_assert(MFMA_MIN > VEC_SMALL_T && MFMA_MIN_WIDE > VEC_SMALL_T,
              "batches with smaller vector items have no matrix-core tiles");
template <int FMT, int BN, int VR>
__global__ __launch_bounds__(256, (FFN_WG_PER_CU<FMT, BN>)) void ffn_up_kernel(LayerArgs a) {
  __shared__ FfnKernelSmem<FMT, BN> sm;
  // matrix-core items: mf_up_chunks(BN) per tile; vector-path items: D_FF / VR per tile
  const int n_all = a.ctl[CTL_N_UP], n_mf = a.ctl[CTL_N_UP_MF];
  constexpr int UC = (BN > 0) ? mf_up_chunks(BN) : 1;
  const int base = (n_mf / UC) * (D_FF / VR);
  if constexpr (BN == 128 && FMT == FMT_BF16) {
    mfma_up_bf16_seq<BN>(a, blockIdx.x, gridDim.x, n_mf, sm.mf);
  } else if constexpr (BN > 0) {
    for (int i = blockIdx.x; i < n_mf; i += gridDim.x) {
      const Item item = fetch_item(a.tiles, mf_item(i, n_mf, UC), UC);
      const bool sh = item_shared(item.head);
      mfma_up<FMT, BN>(a, sel_qmat(sh, a.sh_gate, a.gate), sel_qmat(sh, a.sh_up, a.up), sh ? 0 : item_expert(item.head),
                       item_tokens(item), item_chunk(item.head) * (D_FF / UC), sm.mf);
    }
  }
  up_stream<FMT, VR>(a, base, n_all - base, n_mf, sm.gv, blockIdx.x, gridDim.x);
}

template <int FMT, int BN, int VDR>
__global__ __launch_bounds__(256, (FFN_WG_PER_CU<FMT, BN>)) void ffn_down_kernel(LayerArgs a) {
  __shared__ FfnKernelSmem<FMT, BN> sm;
  const int n_all = a.ctl[CTL_N_DN], n_mf = a.ctl[CTL_N_DN_MF];
  if constexpr (BN > 0 && FMT == FMT_BF16) {
    const int G = mf_grid(n_mf, gridDim.x);
    if ((int)blockIdx.x < G) mfma_down_bf16_seq<BN>(a, blockIdx.x, G, n_mf, sm.mf);
  } else if constexpr (BN > 0) {
    const int G = mf_grid(n_mf, gridDim.x);
    for (int i = blockIdx.x; i < n_mf && (int)blockIdx.x < G; i += G) {
      const Item item = fetch_item(a.tiles, mf_item(i, n_mf, N_DN_CHUNKS), N_DN_CHUNKS);
      const bool sh = item_shared(item.head);
      mfma_down<FMT, BN>(a, sel_qmat(sh, a.sh_down, a.down), sh ? 0 : item_expert(item.head), item_tokens(item),
                         item_chunk(item.head) * DN_ROWS, sm.mf);
    }
  }
  const int base = (n_mf / N_DN_CHUNKS) * (D_MODEL / VDR);
  down_stream<FMT, VDR>(a, base, n_all - base, n_mf, sm.gv, blockIdx.x, gridDim.x);
}

// Workgroups of `kernel` that fit on one CU at once (the persistent kernels are
// launched with exactly the resident count, so none waits for a free slot).
template <typename Kern>
int resident_per_cu(Kern kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

template <int FMT, int BN, int VR, int VDR>
hipError_t launch_ffn_var(const LayerArgs& a, bool up, int n_cu, int max_wgs, hipStream_t s) {
  static const int occ_up = resident_per_cu(ffn_up_kernel<FMT, BN, VR>);
  static const int occ_dn = resident_per_cu(ffn_down_kernel<FMT, BN, VDR>);
  // Kernels with matrix-core tiles run at most MF_WG_PER_CU workgroups per CU:
  // with a third one resident the 256-token NVFP4 layer took 89 instead of 78
  // us (its tile items then share a CU three ways); the vector-only kernels
  // take every resident slot (capped at two they lost 3 us at 64 tokens).
  const int occ = up ? occ_up : occ_dn;
  int grid = n_cu * (BN > 0 ? min(occ, MF_WG_PER_CU) : occ);
  if (max_wgs < grid) grid = max_wgs;
  if (grid < 1) return hipSuccess;
  if (up) hipLaunchKernelGGL((ffn_up_kernel<FMT, BN, VR>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_down_kernel<FMT, BN, VDR>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Matrix-core tiles exist only for buckets (or the shared expert) of
// mfma_min(T) or more tokens, so below that the leaner kernel runs; above, the
// kernel for the batch's tile width.
// The vector item sizes follow vec_up_rows / vec_dn_rows of the batch.
static_assert(vec_up_rows(1) == 16 && vec_up_rows(2) == 32 && vec_up_rows(VEC_SMALL_T) == 32 &&
                  vec_up_rows(VEC_SMALL_T + 1) == UP_ROWS && vec_dn_rows(VEC_SMALL_T) == 128 &&
                  vec_dn_rows(VEC_SMALL_T + 1) == DN_ROWS,
              "the launch below instantiates these item sizes");
template <int FMT>
hipError_t launch_ffn_fmt(const LayerArgs& a, bool up, int n_cu, int max_wgs, hipStream_t s) {
  if (!batch_mfma(a.T)) {
    if (a.T <= 1) return launch_ffn_var<FMT, 0, 16, 128>(a, up, n_cu, max_wgs, s);
    if (a.T <= VEC_SMALL_T) return launch_ffn_var<FMT, 0, 32, 128>(a, up, n_cu, max_wgs, s);
    return launch_ffn_var<FMT, 0, UP_ROWS, DN_ROWS>(a, up, n_cu, max_wgs, s);
  }
  return mfma_bn(a.T) == 64 ? launch_ffn_var<FMT, 64, UP_ROWS, DN_ROWS>(a, up, n_cu, max_wgs, s)
                            : launch_ffn_var<FMT, 128, UP_ROWS, DN_ROWS>(a, up, n_cu, max_wgs, s);
}

hipError_t launch_ffn(const LayerArgs& a, bool up, int n_cu, int max_wgs, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: return launch_ffn_fmt<FMT_Q4_1>(a, up, n_cu, max_wgs, s);
    case FMT_NVFP4: return launch_ffn_fmt<FMT_NVFP4>(a, up, n_cu, max_wgs, s);
    default: return launch_ffn_fmt<FMT_BF16>(a, up, n_cu, max_wgs, s);
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
__device__ inline void combine_token(const LayerArgs& a, int t) {
  const int K = a.K;
  const int i0 = 8 * threadIdx.x;
  // every load is issued before the first sum: the weights and the rows (y
  // rows are slots, t K + j, so that no lookup of bucket positions comes first)
  int pos[MAX_K];
  float wj[MAX_K];
#pragma unroll
  for (int j = 0; j < MAX_K; ++j) {
    pos[j] = t * K + j;
    wj[j] = (j < K) ? a.w[(size_t)t * K + j] : 0.f;
  }
  // (fp32 rows, or bf16 rows for bf16 weights: the branch is uniform)
  const bool ybf = a.fmt == FMT_BF16;
  float4 v[MAX_K + 1][2];
#pragma unroll
  for (int j = 0; j <= MAX_K; ++j) {
    const bool sh = (j == MAX_K);
    if (sh ? a.n_shared != 0 : j < K) {
      const size_t off = (size_t)(sh ? a.S + t : pos[j]) * D_MODEL + i0;
      if (ybf) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.y) + off);
        v[j][0] = make_float4(__uint_as_float(q[0] << 16), __uint_as_float(q[0] & 0xFFFF0000u),
                              __uint_as_float(q[1] << 16), __uint_as_float(q[1] & 0xFFFF0000u));
        v[j][1] = make_float4(__uint_as_float(q[2] << 16), __uint_as_float(q[2] & 0xFFFF0000u),
                              __uint_as_float(q[3] << 16), __uint_as_float(q[3] & 0xFFFF0000u));
      } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.y) + off);
        v[j][0] = p[0];
        v[j][1] = p[1];
      }
    }
  }
  float o[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = 0.f;
#pragma unroll
  for (int j = 0; j <= MAX_K; ++j) {
    const bool sh = (j == MAX_K);
    if (sh ? a.n_shared == 0 : j >= K) continue;
    const float c = sh ? a.shared_scale : wj[j];
    o[0] += c * v[j][0].x; o[1] += c * v[j][0].y; o[2] += c * v[j][0].z; o[3] += c * v[j][0].w;
    o[4] += c * v[j][1].x; o[5] += c * v[j][1].y; o[6] += c * v[j][1].z; o[7] += c * v[j][1].w;
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

__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a) { combine_token(a, blockIdx.x); }

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

// ======================================================================================
// Output head: logits[t][v] = sum_k x[t][k] W[v][k] over a vocabulary of V rows of
// D_MODEL columns.  The review ("The quantisation recipe is the most transferable
// part") stores this head in 4 bits because, with 2.5 B active parameters, it is a
// large share of the bytes each token reads.
//
// Up to 4 tokens it is a streaming GEMV on the vector path's units: persistent
// workgroups over items of HEAD_ROWS rows (a wave takes 16: two pairs of 4-row
// groups), the 4 tokens in LDS in operand order, and each wave's ring of weight
// loads running on from one item into the next; three workgroups per CU.
// ======================================================================================
constexpr int HEAD_ROWS = 64;
// three workgroups per CU: 35.2-35.5 against 36.7 us for one token (two per CU)
constexpr int HEAD_WG_PER_CU = 3;

template <int FMT>
__global__ __launch_bounds__(256, HEAD_WG_PER_CU) void head_kernel(HeadArgs a) {
  __shared__ MvSmem sm;
  using G = GV<FMT>;
  // unit u of an item: pair p = u / 8 of 4-row groups, K-quarter q = (u / 2) % 4,
  // group m = u % 2 of the pair; lane (b, j) reads chunk 16 q + b of row
  // r0 + 8 p + 4 m + j (clamped into the vocabulary; rows past it are read
  // again and not stored)
  constexpr int D = MV_UP_RING<FMT>, NU = 2 * 8;
  static_assert(NU % D == 0 && HEAD_ROWS == 4 * 16, "4 waves x 2 pairs of 4-row groups per item");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, b = lane >> 2;
  const int n = ceil_div(a.V, HEAD_ROWS), G_ = (int)gridDim.x;
  int c = blockIdx.x;
  if (c >= n) return;
  auto first_row = [&](int cc) { return cc * HEAD_ROWS + wave * (HEAD_ROWS / 4); };
  // first row of load u's 4-row group (wave-uniform) and the lane's row offset
  // from it, both clamped into the vocabulary
  auto group_base = [&](int r0_, int u) { return min(r0_ + 8 * (u >> 3) + 4 * (u & 1), a.V - 1); };
  auto lane_sub = [&](int base) { return (uint32_t)min(j, a.V - 1 - base); };
  // 4-bit formats: the codes ride in the ring; the scales of a row group's 4
  // K-quarters (adjacent in storage) come in one load with the group's first
  // unit and are handed to each unit as it is used
  constexpr bool S4 = FMT != FMT_BF16;
  static_assert(!S4 || D == 8, "scale loads follow the ring's 8-load row groups");
  auto load_unit = [&](int r0_, int u) {
    const int base = group_base(r0_, u);
    if constexpr (S4) return G::template load_codes<true>(a.w, (size_t)base, lane_sub(base), 16 * ((u >> 1) & 3) + b, D_MODEL);
    else return G::template load<true>(a.w, (size_t)base, lane_sub(base), 16 * ((u >> 1) & 3) + b, D_MODEL);
  };
  auto load_sc = [&](int r0_, int u) {
    const int base = group_base(r0_, u);
    return G::template load_scales4<true>(a.w, (size_t)base, lane_sub(base), (uint32_t)b);
  };
  int r0 = first_row(c);
  typename G::Raw ring[D];
  typename G::Scales4 s4c[2] = {}, s4n[2] = {};  // scales of the current / next pair, row group m
#pragma unroll
  for (int i = 0; i < D; ++i) ring[i] = load_unit(r0, i);
  if constexpr (S4) {
    s4c[0] = load_sc(r0, 0);
    s4c[1] = load_sc(r0, 1);
  }
  {  // the tokens into LDS (zeros past T): a thread per (token, chunk)
    const int t = (int)threadIdx.x >> 6, cc = (int)threadIdx.x & 63;
    MvStage st;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.v[i] = u32x4{0u, 0u, 0u, 0u};
    if (t < a.T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st.v[i] = ld16<false>(a.x + (size_t)t * D_MODEL + 32 * cc + 8 * i);
    }
    mv_stage_store<FMT, true>(st, sm, 0);  // wave t holds token t's whole row: its scale too
  }
  __syncthreads();
  const float ts = (FMT == FMT_NVFP4) ? a.w.ts[0] : 1.f;
  // after a pair's reduction, lanes with bit 2 clear hold row group 2 p + bit 5
  // of token 2 * bit 4 + bit 3, row j
  const int my_t = ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
  const float tsc = OPER_F16<FMT> ? ts * sm.isc[0][my_t] : ts;  // with the token's inverse scale
#pragma unroll 1
  for (;;) {
    const int nc = c + G_;
    const bool has_next = nc < n;
    const int nr0 = has_next ? first_row(nc) : r0;
    f32x4 acc[2] = {}, negK = {}, S = {};
    uint32_t xq[16];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int p = u >> 3, q = (u >> 1) & 3, m = u & 1;
      if (m == 0) {
        mv_acts<FMT>(sm, 0, 16 * q + b, j, xq, negK, S);
        if (q == 0) acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      typename G::Raw cur = ring[u % D];
      if constexpr (S4) G::set_scale(cur, s4c[m], q);
      const int un = u + D;  // the load issued now
      if (un < NU) {
        ring[u % D] = load_unit(r0, un);
        if (S4 && ((un >> 1) & 3) == 0) s4n[m] = load_sc(r0, un);
      } else if (has_next) {
        ring[u % D] = load_unit(nr0, un - NU);
        if (S4 && (((un - NU) >> 1) & 3) == 0) s4n[m] = load_sc(nr0, un - NU);
      }
      MV<FMT>::unit(cur, xq, negK, S, acc[m]);
      if (u % 8 == 7) {
        if constexpr (S4) {
          s4c[0] = s4n[0];
          s4c[1] = s4n[1];
        }
        const float v = mv_reduce8(acc[0], acc[1]) * tsc;
        const int row = r0 + 8 * p + 4 * ((lane >> 5) & 1) + j, t = my_t;
        if ((lane & 4) == 0 && row < a.V && t < a.T) a.logits[(size_t)t * a.V + row] = v;
      }
    }
    if (!has_next) break;
    c = nc;
    r0 = nr0;
  }
}

// ---- the head on the matrix cores (batches of more than 4 tokens) -----------------
// With more than one 4-token group the 4x4x4 products, not the weight stream,
// set the vector kernel's pace.  Here the 16x16x32 MFMA multiplies 16 tokens
// (A, from LDS) by 16 vocabulary rows (B, decoded in registers): lane (r, g)
// holds row r of a 16-row block and k-group g, and each of its 16-byte weight
// loads is one 32-element block that feeds 4 MFMAs per 16-token tile.  A pass
// keeps NT tiles (16 NT tokens) resident in LDS for all of its items; a wave
// takes RB blocks of 16 rows, its ring holds D loads, and an item is the
// waves' rows.  K-step z = 4 i + a (a < 4) of a row reads block 16 i + 4 a + g:
// four steps in a row read 256 contiguous bytes of it, and the scales of the
// steps with one a are adjacent in storage (one load per a, per item).  The
// x tile: [block][token][16-byte sub-block s XOR (token / 4) mod 4] in the weights'
// decode order, so that the 16 lanes of a k-group read 16 tokens without bank
// conflicts.  Batches beyond 32 tokens take passes of 32.  Item c is row chunk
// rc of pass tp, numbered so that the passes of a row chunk fall on one XCD
// (workgroup id mod 8 under round-robin dispatch, with the grid a multiple of 8)
// and on workgroups that run at the same time, where their repeated reads of the
// chunk can meet in that XCD's L2.
template <int NT> constexpr int HMF_W = NT == 1 ? 4 : 8;  // waves per workgroup
template <int NT> constexpr int HMF_RB = NT == 1 ? 2 : 1;  // 16-row blocks per wave
// weight loads in flight per wave (a bf16 load is 64 bytes a lane, a 4-bit one 16)
template <int FMT> constexpr int HMF_D = FMT == FMT_BF16 ? 4 : 8;
template <int NT> constexpr int HMF_ROWS = HMF_W<NT> * 16 * HMF_RB<NT>;  // rows per item
template <int NT> struct HeadMfSmem {
  u32x4 x[MV_CHUNKS][16 * NT][4];
  float isc[16 * NT];  // 4-bit formats: inverse activation scale per token of the pass
};

template <int FMT> __device__ inline f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (OPER_F16<FMT>)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

template <int FMT, int NT>
__global__ __launch_bounds__(64 * HMF_W<NT>, NT == 1 ? 2 : 1) void head_mf_kernel(HeadArgs a) {
  constexpr int W = HMF_W<NT>, RB = HMF_RB<NT>, D = HMF_D<FMT>, NU = 16 * RB, TT = 16 * NT, ROWS = HMF_ROWS<NT>;
  static_assert(NU % D == 0, "the ring holds whole items");
  __shared__ HeadMfSmem<NT> sm;
  using G = GV<FMT>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int ntp = ceil_div(a.T, TT), nrc = ceil_div(a.V, ROWS);
  // items: XCD slot c % 8, then k = c / 8 -> row chunk 8 (k / ntp) + slot, pass k % ntp
  const int n = 8 * ntp * ceil_div(nrc, 8), G_ = (int)gridDim.x;
  int c = blockIdx.x;
  if (c >= n) return;
  auto item_tp = [&](int cc) { return (cc >> 3) % ntp; };
  auto first_row = [&](int cc) { return (8 * ((cc >> 3) / ntp) + (cc & 7)) * ROWS + wave * 16 * RB; };
  // unit u: k-step z = u / RB of row block rb = u % RB; rows clamped into the
  // vocabulary (read again, never stored)
  auto row_base = [&](int r0_, int rb) { return min(r0_ + 16 * rb, a.V - 1); };
  auto lane_sub = [&](int base) { return (uint32_t)min(r16, a.V - 1 - base); };
  auto block_of = [&](int z) { return 16 * (z >> 2) + 4 * (z & 3) + g; };
  constexpr bool S4 = FMT != FMT_BF16;
  auto load_unit = [&](int r0_, int u) {
    const int base = row_base(r0_, u % RB);
    if constexpr (S4) return G::template load_codes<true>(a.w, (size_t)base, lane_sub(base), block_of(u / RB), D_MODEL);
    else return G::template load<true>(a.w, (size_t)base, lane_sub(base), block_of(u / RB), D_MODEL);
  };
  // scales of blocks 4 s + g + 16 i (i < 4): the steps z = 4 i + s of row block rb
  typename G::Scales4 sc[RB][4], sn[RB][4];
  auto load_scales = [&](int r0_, typename G::Scales4 (&dst)[RB][4]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int base = row_base(r0_, rb);
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_)
        dst[rb][s_] = G::template load_scales4<true>(a.w, (size_t)base, lane_sub(base), (uint32_t)(4 * s_ + g));
    }
  };
  // the pass's tokens TT tp .. into LDS (zeros past T): thread (token, block)
  // pairs, TT / W per thread, all loads in flight before the stores
  static_assert(TT % W == 0, "whole tokens per wave");
  auto stage = [&](int tp) {
    const int blk = (int)threadIdx.x & 63, t0 = (int)threadIdx.x >> 6;
    u32x4 v[TT / W][4];
#pragma unroll
    for (int k = 0; k < TT / W; ++k) {
      const int t = TT * tp + t0 + W * k;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[k][i] = (t < a.T) ? ld16<false>(a.x + (size_t)t * D_MODEL + 32 * blk + 8 * i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < TT / W; ++k) {
      const int tl = t0 + W * k;
      float sc = 1.f;
      if constexpr (OPER_F16<FMT>) {  // the wave holds the token's whole row: its scale
        uint32_t m = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, bf16_absmax8(v[k][i]));
        sc = pow2_scale(wave_max_u32(m) << 16);
        if (blk == 0) sm.isc[tl] = pow2_inv(sc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t e[4] = {v[k][i][0], v[k][i][1], v[k][i][2], v[k][i][3]}, o[4];
        if constexpr (OPER_F16<FMT>) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = bf16x2_to_f16x2(e[q], sc);
        }
        if constexpr (FMT == FMT_Q4_1) q4_order(e[0], e[1], e[2], e[3], o);
        else {
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = e[q];
        }
        sm.x[blk][tl][i ^ ((tl >> 2) & 3)] = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  };
  int tp = item_tp(c), r0 = first_row(c);
  typename G::Raw ring[D];
#pragma unroll
  for (int i = 0; i < D; ++i) ring[i] = load_unit(r0, i);
  if constexpr (S4) load_scales(r0, sc);
  stage(tp);
  __syncthreads();
  const float ts = (FMT == FMT_NVFP4) ? a.w.ts[0] : 1.f;
  const int swz = (r16 >> 2) & 3;
#pragma unroll 1
  for (;;) {
    const int nc = c + G_;
    const bool has_next = nc < n;
    const int nr0 = has_next ? first_row(nc) : r0;
    f32x4 acc[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[rb][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < 16; ++z) {
      u32x4 xa[NT][4];  // A operands: tokens 16 tt + r16 of block block_of(z), sub-blocks s
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_) xa[tt][s_] = sm.x[block_of(z)][16 * tt + r16][s_ ^ swz];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int u = z * RB + rb;
        typename G::Raw cur = ring[u % D];
        if constexpr (S4) G::set_scale(cur, sc[rb][z & 3], z >> 2);
        const int un = u + D;  // the load issued now
        if (un < NU) {
          ring[u % D] = load_unit(r0, un);
        } else if (has_next) {
          ring[u % D] = load_unit(nr0, un - NU);
          if (S4 && un == NU) load_scales(nr0, sn);
        }
        uint32_t w[16];
        G::decode(cur, w);
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            acc[rb][tt] = mfma16<FMT>(xa[tt][s_], u32x4{w[4 * s_], w[4 * s_ + 1], w[4 * s_ + 2], w[4 * s_ + 3]},
                                      acc[rb][tt]);
      }
    }
    // acc[rb][tt][j]: token 16 tt + 4 g + j of the pass, row r0 + 16 rb + r16
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = r0 + 16 * rb + r16;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = TT * tp + 16 * tt + 4 * g + j;
          const float tsc = OPER_F16<FMT> ? ts * sm.isc[16 * tt + 4 * g + j] : ts;
          if (row < a.V && t < a.T) a.logits[(size_t)t * a.V + row] = acc[rb][tt][j] * tsc;
        }
    }
    if (!has_next) break;
    if constexpr (S4) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int s_ = 0; s_ < 4; ++s_) sc[rb][s_] = sn[rb][s_];
    }
    const int ntpc = item_tp(nc);
    if (ntpc != tp) {  // another pass: every wave is done with the tile before it is replaced
      __syncthreads();
      stage(ntpc);
      __syncthreads();
      tp = ntpc;
    }
    c = nc;
    r0 = nr0;
  }
}

template <int FMT, int NT> hipError_t launch_head_mf(const HeadArgs& a, int n_cu, hipStream_t s) {
  const int ntp = ceil_div(a.T, 16 * NT), nrc = ceil_div(a.V, HMF_ROWS<NT>);
  const int n = 8 * ntp * ceil_div(nrc, 8);
  int grid = n_cu * (NT == 1 ? 2 : 1);
  grid -= grid % 8;
  if (grid < 8) grid = 8;
  if (n < grid) grid = n;
  hipLaunchKernelGGL((head_mf_kernel<FMT, NT>), dim3(grid), dim3(64 * HMF_W<NT>), 0, s, a);
  return hipGetLastError();
}

template <int FMT> hipError_t launch_head_vec(const HeadArgs& a, int n_cu, hipStream_t s) {
  const int n = ceil_div(a.V, HEAD_ROWS);
  int grid = n_cu * HEAD_WG_PER_CU;
  if (n < grid) grid = n;
  hipLaunchKernelGGL(head_kernel<FMT>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMT> hipError_t launch_head_fmt(const HeadArgs& a, int n_cu, hipStream_t s) {
  if (a.T <= GV_GROUP) return launch_head_vec<FMT>(a, n_cu, s);
  return a.T <= 16 ? launch_head_mf<FMT, 1>(a, n_cu, s) : launch_head_mf<FMT, 2>(a, n_cu, s);
}

hipError_t launch_head(const HeadArgs& a, int n_cu, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: return launch_head_fmt<FMT_Q4_1>(a, n_cu, s);
    case FMT_NVFP4: return launch_head_fmt<FMT_NVFP4>(a, n_cu, s);
    default: return launch_head_fmt<FMT_BF16>(a, n_cu, s);
  }
}

}  // namespace moe
