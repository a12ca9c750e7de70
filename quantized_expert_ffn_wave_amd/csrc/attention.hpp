// Decode attention: shapes and kernel arguments shared by the attention
// kernels and the C ABI (one new token per sequence).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Decode attention (one new token per sequence): heads, dimension, arguments.
constexpr int ATTN_HQ = 32, ATTN_HK = 4, ATTN_D = 128;
struct AttnArgs {
  const uint16_t* q;        // bf16 [B][HQ][D] new token, before norm and rotation
  const uint16_t* k;        // bf16 [B][HK][D]
  const uint16_t* v;        // bf16 [B][HK][D]
  const uint16_t* q_gain;   // bf16 [D]
  const uint16_t* k_gain;   // bf16 [D]
  const float* sinks;       // [HQ] or null
  const int32_t* pos;       // [B] position of the new token
  uint16_t* k_cache;        // bf16 [B][HK][cap][D]
  uint16_t* v_cache;        // bf16 [B][HK][D][cap] (transposed)
  uint16_t* qbuf;           // bf16 [B][HQ][D] prepared q (workspace)
  float* part_o;            // [B][HQ][splits][D] unnormalised partial outputs (workspace)
  float* part_ml;           // [B][HQ][splits][2] running maximum (log2 domain) and sum (workspace)
  uint16_t* out;            // bf16 [B][HQ][D]
  int cap, window, rope, splits;
  float eps;
  // rotation frequencies: theta^(-d/64) = rot_32^(d / 32) * rot_g[(d / 8) % 4] * rot_e[d % 8]
  double rot_e[8], rot_g[4], rot_32;
};
hipError_t launch_attn(const AttnArgs& a, int B, hipStream_t s);

}  // namespace moe
