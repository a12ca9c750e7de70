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

enum Fmt : int { FMT_BF16 = 0, FMT_Q4_1 = 1, FMT_NVFP4 = 2 };

// ---- work items ---------------------------------------------------------------
// A work item names (expert, token tile, row chunk, path).  Expert value
// MAX_E means the shared expert.  The bucket kernel writes the lists; the FFN
// kernels decode them.
constexpr uint32_t ITEM_MFMA = 0x80000000u;
__host__ __device__ inline uint32_t make_item(int e, int chunk, int tile, bool mfma) {
  return (uint32_t)e | ((uint32_t)chunk << 9) | ((uint32_t)tile << 16) | (mfma ? ITEM_MFMA : 0u);
}
__device__ inline int item_expert(uint32_t it) { return (int)(it & 511u); }
__device__ inline int item_chunk(uint32_t it) { return (int)((it >> 9) & 127u); }
__device__ inline int item_tile(uint32_t it) { return (int)((it >> 16) & 0x7FFFu); }
__device__ inline bool item_mfma(uint32_t it) { return (it & ITEM_MFMA) != 0; }

// GEMV path: buckets of at most GEMV_MAX tokens.  Rows per item.
constexpr int GEMV_MAX = 4;
constexpr int UP_GEMV_ROWS = 16;    // gate/up row pairs per GEMV item (4 waves x 4)
constexpr int DN_GEMV_ROWS = 64;    // down rows per GEMV item (4 waves x 16)
// MFMA path: token tile and row chunk per item.
constexpr int MFMA_BN = 64;         // tokens per MFMA item (two 32-token tiles)
constexpr int UP_MFMA_ROWS = 64;    // gate/up row pairs per MFMA item (4 waves x 16)
constexpr int DN_MFMA_ROWS = 128;   // down rows per MFMA item (4 waves x 32)

// ---- control block and pointers handed to kernels -----------------------------
enum Ctl : int { CTL_N_UP = 0, CTL_N_DN = 1, CTL_WORDS = 16 };

struct QMat {
  const uint8_t* codes;   // q4_1/nvfp4 nibbles or bf16 elements
  const void* scales;     // q4_1 half2 {d, m}; nvfp4 E4M3 bytes
  const float* ts;        // nvfp4 per-matrix scale
};

// Everything one layer forward needs on the device (passed by value).
struct LayerArgs {
  int T, E, K, S, n_shared, renorm, fmt, ks;  // ks = router K-splits
  float shared_scale;
  const uint16_t* x;        // bf16 [T][D_MODEL]
  const uint16_t* router_w; // bf16 [E][D_MODEL]
  const float* router_b;    // [E] or null
  QMat gate, up, down, sh_gate, sh_up, sh_down;
  // workspace
  float* logit_part;        // [ks][T][E]
  float* logits;            // [T][E] (written only if requested)
  int32_t* ids;             // [T][K]
  float* w;                 // [T][K]
  int32_t* counts;          // [E]
  int32_t* offsets;         // [E+1]
  int32_t* perm;            // [S]
  int32_t* inv_perm;        // [S]
  uint32_t* items_up;       // work list, gate/up
  uint32_t* items_dn;       // work list, down
  int32_t* ctl;             // [CTL_WORDS]
  _Float16* h;              // [S + n_shared*T][D_FF] SwiGLU output, fp16
  float* y;                 // [S + n_shared*T][D_MODEL] expert outputs, fp32
  int max_items_up, max_items_dn;
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

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

constexpr int WAVE = 64;

}  // namespace moe

// Host-side launchers (defined in the .hip files, called by the ABI layer).
namespace moe {
hipError_t launch_router(const LayerArgs& a, hipStream_t s);
hipError_t launch_topk(const LayerArgs& a, bool write_logits, hipStream_t s);
hipError_t launch_bucket(const LayerArgs& a, hipStream_t s);
hipError_t launch_ffn_up(const LayerArgs& a, int grid, hipStream_t s);
hipError_t launch_ffn_down(const LayerArgs& a, int grid, hipStream_t s);
hipError_t launch_combine(const LayerArgs& a, uint16_t* out_bf16, hipStream_t s);
// stack glue: r (fp32 [T][D]) and xn (bf16 [T][D])
hipError_t launch_stack_init(const uint16_t* x, float* r, uint16_t* xn, int T, float eps, hipStream_t s);
hipError_t launch_combine_stack(const LayerArgs& a, float* r, uint16_t* xn_next, uint16_t* y_rec, uint16_t* x_final,
                                float eps, hipStream_t s);
}  // namespace moe
