// Shared device/host definitions of the gfx950 MoE-layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- fixed problem shape this build has kernels for -------------------------
constexpr int D_MODEL = 2048;  // hidden size
constexpr int D_FF = 512;      // expert width (routed and shared)
constexpr int MAX_E = 256;     // routed experts
constexpr int MAX_K = 8;       // experts per token
constexpr int SHARED_ID = MAX_E;  // expert id of the shared expert in the work lists
constexpr int HSLOTS = D_FF / 16; // slots of a row's |h| maximum (16 columns each)

enum Fmt : int { FMT_BF16 = 0, FMT_Q4_1 = 1, FMT_NVFP4 = 2 };

// ---- work decomposition ---------------------------------------------------------
// A bucket of m tokens is split into token groups of GV_GROUP (vector path) when
// m < mfma_min(T), else into token tiles of mfma_bn(T) tokens (matrix-core
// path): 64 in batches of up to MFMA_WIDE_T tokens, 128 in larger ones (where
// buckets are large, a wider tile streams an expert's weights fewer times;
// where they are not, narrower tiles make more and shorter items).  The
// threshold is MFMA_MIN up to MFMA_MID_T tokens, where most buckets are small
// and a tile item is slower than the vector items it replaces, and
// MFMA_MIN_WIDE above, where mid-size buckets would otherwise stream their
// expert's weights once per 4 tokens.  Both paths cover
// UP_ROWS gate/up row pairs (vector path; matrix-core path: D_FF / mf_up_chunks
// of the tile width), or DN_ROWS down rows, per work item.
constexpr int GV_GROUP = 4;
constexpr int MFMA_MIN = 65;
constexpr int MFMA_MIN_WIDE = 16;
constexpr int MFMA_MID_T = 128;
constexpr int MFMA_WIDE_T = 256;
constexpr int UP_ROWS = 64;
constexpr int DN_ROWS = 256;
constexpr int N_UP_CHUNKS = D_FF / UP_ROWS;      // 8
constexpr int N_DN_CHUNKS = D_MODEL / DN_ROWS;   // 8
// In batches of up to VEC_SMALL_T tokens (7 experts a token, no matrix-core
// tiles) the standard vector items would leave most workgroups idle, so they
// are cut smaller: gate/up items of 16 row pairs for one token and 32 up to
// VEC_SMALL_T, down items of 128 rows.
constexpr int VEC_SMALL_T = 8;
__host__ __device__ constexpr int vec_up_rows(int T) { return T <= 1 ? 16 : T <= VEC_SMALL_T ? 32 : UP_ROWS; }
__host__ __device__ constexpr int vec_dn_rows(int T) { return T <= VEC_SMALL_T ? 128 : DN_ROWS; }
__host__ __device__ constexpr int vec_up_chunks(int T) { return D_FF / vec_up_rows(T); }
__host__ __device__ constexpr int vec_dn_chunks(int T) { return D_MODEL / vec_dn_rows(T); }

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int mfma_bn(int T) { return T > MFMA_WIDE_T ? 128 : 64; }
// gate/up items per matrix-core tile of width bn: 128 row pairs each for
// 128-token tiles, 64 for 64-token ones
__host__ __device__ constexpr int mf_up_chunks(int bn) { return bn == 128 ? 4 : 8; }
// path and token groups/tiles of a bucket of m tokens in a batch of T tokens
__host__ __device__ constexpr int mfma_min(int T) { return T > MFMA_MID_T ? MFMA_MIN_WIDE : MFMA_MIN; }
__host__ __device__ constexpr bool bucket_mfma(int m, int T) { return m >= mfma_min(T); }
__host__ __device__ inline int bucket_tiles(int m, int T) {
  return m <= 0 ? 0 : (bucket_mfma(m, T) ? ceil_div(m, mfma_bn(T)) : ceil_div(m, GV_GROUP));
}
// The shared expert (all T tokens) takes tiles from MFMA_MIN tokens on at every
// batch size: a tile holding a few dozen tokens is slower than its vector groups.
__host__ __device__ constexpr bool shared_mfma(int T) { return T >= MFMA_MIN; }
__host__ __device__ inline int shared_tiles(int T) {
  return T <= 0 ? 0 : (shared_mfma(T) ? ceil_div(T, mfma_bn(T)) : ceil_div(T, GV_GROUP));
}
// whether a batch of T tokens can have matrix-core tiles at all
__host__ __device__ inline bool batch_mfma(int T) { return bucket_mfma(T, T) || shared_mfma(T); }

// Work item (16 bytes, so that a kernel needs one load to start streaming):
//   head: expert (9 bits; SHARED_ID = the shared expert) | row chunk << 9 (5 bits) |
//         token count << 14 (8 bits) | matrix-core path << 31
//   p0:   first bucket position (routed) or first token (shared); the expert
//         output rows of the item are p0.. (routed) or S + p0.. (shared)
//   t01, t23: token ids of a vector-path item (16 bits each)
struct Item {
  uint32_t head, p0, t01, t23;
};
constexpr uint32_t ITEM_MFMA = 0x80000000u;
__host__ __device__ inline uint32_t item_head(int e, int chunk, int cnt, bool mfma) {
  return (uint32_t)e | ((uint32_t)chunk << 9) | ((uint32_t)cnt << 14) | (mfma ? ITEM_MFMA : 0u);
}
__device__ inline int item_expert(uint32_t h) { return (int)(h & 511u); }
__device__ inline bool item_shared(uint32_t h) { return item_expert(h) == SHARED_ID; }
__device__ inline int item_chunk(uint32_t h) { return (int)((h >> 9) & 31u); }
__device__ inline int item_count(uint32_t h) { return (int)((h >> 14) & 255u); }
__device__ inline bool item_mfma(uint32_t h) { return (h & ITEM_MFMA) != 0; }

// ---- control block ------------------------------------------------------------------
enum Ctl : int { CTL_N_UP = 0, CTL_N_DN = 1, CTL_N_UP_MF = 2, CTL_N_DN_MF = 3, CTL_WORDS = 16 };
// hand-off words of the persistent decode path (workspace; cleared by its first launch)
enum DecSync : int { DEC_SYNC_TOPK = 0, DEC_SYNC_B1 = 1, DEC_SYNC_B2 = 2, DEC_SYNC_B3 = 3, DEC_SYNC_TIMEOUT = 15,
                     DEC_SYNC_WORDS = 16 };

struct QMat {
  const uint8_t* codes;   // q4_1/nvfp4 nibbles or bf16 elements
  const void* scales;     // q4_1 half2 {d, m}; nvfp4 E4M3 bytes
  const float* ts;        // nvfp4 per-matrix scale
};

// Everything one layer forward needs on the device (passed by value).
struct LayerArgs {
  int T, E, K, S, n_shared, renorm, fmt;
  float shared_scale;
  const uint16_t* x;        // bf16 [T][D_MODEL]
  const uint16_t* router_w; // bf16 [E][D_MODEL]
  const float* router_b;    // [E] or null
  QMat gate, up, down, sh_gate, sh_up, sh_down;
  // workspace
  float* logit_part;        // [8][T][E] router partial sums
  float* logits;            // [T][E] (written only if write_logits)
  int write_logits;
  int32_t* ids;             // [T][K]
  float* w;                 // [T][K]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* perm;            // [S]
  int32_t* inv_perm;        // [S]
  Item* tiles;              // work list: one entry per token tile (row chunk 0)
  int32_t* ctl;             // [CTL_WORDS]
  void* h;                  // [S + n_shared*T][D_FF] SwiGLU output: fp32 for the 4-bit formats, bf16 bits else
  void* y;                  // [S + n_shared*T][D_MODEL] expert outputs, row t K + j for slot j of token t
                            // (S + t for the shared expert): fp32 for the 4-bit formats, bf16 bits
                            // for bf16 weights (whose layer output is bf16 of a 7-term sum of them)
  // 4-bit formats only (their products run on fp16 operands): the power-of-two
  // scale of each token's activations, and per expert-output row the largest
  // |h| of each 16 columns' slot, written by the gate/up item that computes
  // those columns (each slot exactly once per forward) and read by down
  float* xsc;               // [T]
  uint16_t* xq;             // [T][D_MODEL] fp16 bits: x times xsc, in the weights' k order (matrix-core tiles)
  float* hslot;             // [S + n_shared*T][HSLOTS]
  int max_tiles;
  // combine targets
  uint16_t* out;            // bf16 [T][D_MODEL] layer output (single layer), or null
  float* r;                 // fp32 [T][D_MODEL] residual (stack), or null
  uint16_t* y_rec;          // bf16 [T][D_MODEL] record of the layer output (stack), or null
  uint16_t* xn_next;        // bf16 [T][D_MODEL] next layer input (stack), or null
  uint16_t* x_final;        // bf16 [T][D_MODEL] final output (stack, last layer), or null
  float eps;
};

// ---- small helpers ---------------------------------------------------------------
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// silu(g) * u with the hardware reciprocal (1 ulp; the result is stored in 16 bits)
__device__ inline float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// Power-of-two scale for a row of activations whose largest magnitude has the
// fp32 bit pattern `maxbits` (sign clear): the largest element lands in
// [2^14, 2^15), so the row fits fp16 with its full 11-bit precision (the fp16
// maximum is about 2^16).  The exponent is clamped to [-100, 100], which leaves
// all-zero and tiny rows unscaled past 2^100.  Multiplying by it, and by its
// inverse, is exact in fp32.
__device__ inline float pow2_scale(uint32_t maxbits) {
  const int e = (int)(maxbits >> 23);  // biased exponent of the row maximum
  const int k = min(max(141 - e, -100), 100);
  return __uint_as_float((uint32_t)(k + 127) << 23);
}
__device__ inline float pow2_inv(float s) { return __uint_as_float((254u << 23) - __float_as_uint(s)); }

// Lane exchange for the wave-wide maximum: step m pairs lane i with i ^ m
// (m = 4: with 7 - i inside groups of 8, which reaches the same set).
template <int M> __device__ inline uint32_t xchg(uint32_t v) {
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    constexpr int ctrl = (M == 8) ? 0x128 : (M == 4) ? 0x141 : (M == 2) ? 0x4E : 0xB1;
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, false);
  }
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, xchg<32>(v));
  v = max(v, xchg<16>(v));
  v = max(v, xchg<8>(v));
  v = max(v, xchg<4>(v));
  v = max(v, xchg<2>(v));
  v = max(v, xchg<1>(v));
  return v;
}

}  // namespace moe

// Host-side launchers (defined in the .hip files, called by the ABI layer).
namespace moe {
// Output head GEMV: logits[t][v] = sum_k x[t][k] w[v][k], D_MODEL columns.
struct HeadArgs {
  const uint16_t* x;  // bf16 [T][D_MODEL]
  QMat w;             // [V][D_MODEL] in `fmt`
  float* logits;      // fp32 [T][V]
  int T, V, fmt;
};
hipError_t launch_router(const LayerArgs& a, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, hipStream_t s);
hipError_t launch_bucket(const LayerArgs& a, hipStream_t s);
hipError_t launch_combine(const LayerArgs& a, hipStream_t s);
// gate/up (up) or down over the work list (routed and shared experts); at most
// max_wgs workgroups, else as many as are resident on n_cu CUs at once
hipError_t launch_ffn(const LayerArgs& a, bool up, int n_cu, int max_wgs, hipStream_t s);
hipError_t launch_stack_init(const uint16_t* x, float* r, uint16_t* xn, int T, float eps, hipStream_t s);
// persistent decode layer (two launches) for batches of decode_supported(T) tokens
bool decode_supported(int T);
hipError_t launch_decode(const LayerArgs& a, uint32_t* sync, int n_cu, hipStream_t s);
// output head over n_cu compute units
hipError_t launch_head(const HeadArgs& a, int n_cu, hipStream_t s);
// plain streaming read of bytes (a multiple of 16) from src on grid workgroups
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t s);
// matrix-core instructions of one kind (0 f16, 1 bf16, 2 fp8, 3 scaled fp4) only:
// iters x 4 per wave on grid workgroups of 256 threads
hipError_t launch_mfma_rate(int kind, int iters, int grid, float* sink, hipStream_t s);
}  // namespace moe
