// C ABI of the MoE-layer library (declared in include/moe_ffn.h): argument
// validation, workspace layout and kernel sequencing.  No device memory is
// allocated here and nothing synchronises the host.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "common.hpp"
#include "attention.hpp"
#include "probes.hpp"
#include "moe_ffn.h"

// Handle: the checked descriptor and the borrowed weights (no GPU resources).
struct moe_layer {
  moe_layer_desc desc;
  moe_layer_weights w;
  int device;
  int n_cu;
};

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->wfmt < MOE_W_BF16 || d->wfmt > MOE_W_NVFP4) return fail(MOE_ERR_INVALID_ARG, "unknown wfmt %d", d->wfmt);
  if (d->n_experts < 16 || d->n_experts > moe::MAX_E || d->n_experts % 16)
    return fail(MOE_ERR_INVALID_ARG, "n_experts must be a multiple of 16 in [16, 256], got %d", d->n_experts);
  if (d->top_k < 1 || d->top_k > moe::MAX_K || d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, min(8, n_experts)], got %d", d->top_k);
  if (d->n_shared != 0 && d->n_shared != 1) return fail(MOE_ERR_INVALID_ARG, "n_shared must be 0 or 1");
  if (d->renorm_topk != 0 && d->renorm_topk != 1) return fail(MOE_ERR_INVALID_ARG, "renorm_topk must be 0 or 1");
  if (d->max_tokens < 1 || d->max_tokens > 65536)
    return fail(MOE_ERR_INVALID_ARG, "max_tokens must be in [1, 65536], got %d", d->max_tokens);
  if (d->d_model <= 0 || d->d_expert <= 0) return fail(MOE_ERR_INVALID_ARG, "d_model and d_expert must be positive");
  if (d->n_shared && d->d_shared != d->d_expert)
    return fail(MOE_ERR_INVALID_ARG, "d_shared (%d) must equal d_expert (%d)", d->d_shared, d->d_expert);
  if (d->d_model != moe::D_MODEL || d->d_expert != moe::D_FF)
    return fail(MOE_ERR_UNSUPPORTED, "this build has kernels for d_model=%d, d_expert=%d (got %d, %d)", moe::D_MODEL,
                moe::D_FF, d->d_model, d->d_expert);
  return MOE_OK;
}

moe_status check_qmat(const moe_qmat& q, int fmt, const char* name) {
  if (!q.codes || !aligned(q.codes, 16)) return fail(MOE_ERR_INVALID_ARG, "%s.codes is NULL or not 16-byte aligned", name);
  if (fmt == MOE_W_Q4_1 && (!q.scales || !aligned(q.scales, 16)))
    return fail(MOE_ERR_INVALID_ARG, "%s.scales (q4_1 {d,m}) is NULL or not 16-byte aligned", name);
  if (fmt == MOE_W_NVFP4) {
    if (!q.scales || !aligned(q.scales, 8))
      return fail(MOE_ERR_INVALID_ARG, "%s.scales (NVFP4 E4M3) is NULL or not 8-byte aligned", name);
    if (!q.tensor_scale || !aligned(q.tensor_scale, 4))
      return fail(MOE_ERR_INVALID_ARG, "%s.tensor_scale is NULL or not 4-byte aligned", name);
  }
  return MOE_OK;
}

struct WsLayout {
  size_t logit_part, logits, ids, w, counts, offsets, perm, inv_perm, tiles, ctl, h, y, xsc, xq, hslot, sync, total;
  int max_tiles;
};

WsLayout ws_layout(const moe_layer_desc& d, int T) {
  WsLayout L;
  const int E = d.n_experts, K = d.top_k;
  const size_t S = (size_t)T * K, R = S + (size_t)d.n_shared * T;
  // token tiles of the routed buckets, sum_e ceil(m_e / GV_GROUP) <= touched + S / GV_GROUP,
  // plus those of the shared expert
  const int tiles = (int)((S < (size_t)E ? S : (size_t)E) + S / moe::GV_GROUP + 1) +
                    (d.n_shared ? moe::shared_tiles(T) : 0);
  L.max_tiles = tiles;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes > 0 ? bytes : 1); return at; };
  L.logit_part = take(sizeof(float) * 8 * T * E);
  L.logits = take(sizeof(float) * (size_t)T * E);
  L.ids = take(sizeof(int32_t) * S);
  L.w = take(sizeof(float) * S);
  L.counts = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 1));
  L.perm = take(sizeof(int32_t) * S);
  L.inv_perm = take(sizeof(int32_t) * S);
  L.tiles = take(sizeof(moe::Item) * L.max_tiles);
  L.ctl = take(sizeof(int32_t) * moe::CTL_WORDS);
  // SwiGLU output: fp32 for the 4-bit formats (scaled into fp16 by the down
  // kernel with the row's largest |h|), bf16 for bf16 weights
  L.h = take((d.wfmt == MOE_W_BF16 ? sizeof(uint16_t) : sizeof(float)) * R * moe::D_FF);
  // expert outputs: fp32 for the 4-bit formats, bf16 for bf16 weights (the
  // prefill volume: 7 rows of 2048 per token)
  L.y = take((d.wfmt == MOE_W_BF16 ? sizeof(uint16_t) : sizeof(float)) * R * moe::D_MODEL);
  L.xsc = take(sizeof(float) * (size_t)T);
  // 4-bit formats: the scaled fp16 activations the matrix-core tiles read
  // (none where the batch has no tile)
  L.xq = take(d.wfmt == MOE_W_BF16 || !moe::batch_mfma(T) ? 0 : sizeof(uint16_t) * (size_t)T * moe::D_MODEL);
  L.hslot = take(sizeof(float) * moe::HSLOTS * R);
  L.sync = take(sizeof(uint32_t) * moe::DEC_SYNC_WORDS);
  L.total = o;
  return L;
}

moe::QMat qm(const moe_qmat& q) {
  moe::QMat r;
  r.codes = (const uint8_t*)q.codes;
  r.scales = q.scales;
  r.ts = q.tensor_scale;
  return r;
}

moe::LayerArgs make_args(const moe_layer* L, const void* x, int T, char* ws, const WsLayout& W) {
  moe::LayerArgs a;
  memset(&a, 0, sizeof a);
  const moe_layer_desc& d = L->desc;
  a.T = T;
  a.E = d.n_experts;
  a.K = d.top_k;
  a.S = T * d.top_k;
  a.n_shared = d.n_shared;
  a.renorm = d.renorm_topk;
  a.fmt = d.wfmt;
  a.shared_scale = d.shared_scale;
  a.x = (const uint16_t*)x;
  a.router_w = (const uint16_t*)L->w.router_w;
  a.router_b = L->w.router_b;
  a.gate = qm(L->w.gate);
  a.up = qm(L->w.up);
  a.down = qm(L->w.down);
  if (d.n_shared) {
    a.sh_gate = qm(L->w.sh_gate);
    a.sh_up = qm(L->w.sh_up);
    a.sh_down = qm(L->w.sh_down);
  }
  a.logit_part = (float*)(ws + W.logit_part);
  a.logits = (float*)(ws + W.logits);
  a.ids = (int32_t*)(ws + W.ids);
  a.w = (float*)(ws + W.w);
  a.counts = (int32_t*)(ws + W.counts);
  a.offsets = (int32_t*)(ws + W.offsets);
  a.perm = (int32_t*)(ws + W.perm);
  a.inv_perm = (int32_t*)(ws + W.inv_perm);
  a.tiles = (moe::Item*)(ws + W.tiles);
  a.ctl = (int32_t*)(ws + W.ctl);
  a.h = (void*)(ws + W.h);
  a.y = (void*)(ws + W.y);
  a.xsc = (float*)(ws + W.xsc);
  a.xq = (a.fmt != moe::FMT_BF16 && moe::batch_mfma(a.T)) ? (uint16_t*)(ws + W.xq) : nullptr;
  a.hslot = (float*)(ws + W.hslot);
  a.max_tiles = W.max_tiles;
  return a;
}

hipError_t copy_async(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (!dst || bytes == 0) return hipSuccess;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

hipError_t mark(void* const* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess;
}

// One layer on stream s: router, top-k, buckets and work lists, gate/up +
// SwiGLU and down over the routed and shared experts, combine.  Route copies
// (except the output) are enqueued before the combine, which in a stack
// overwrites the layer input.  ev (optional): stage records.
moe_status run_layer(const moe_layer* L, moe::LayerArgs& a, const WsLayout& W, const moe_route_out* route,
                     hipStream_t s, void* const* ev, char* ws = nullptr, bool persistent = false) {
  hipError_t e;
  a.write_logits = (route && route->logits) ? 1 : 0;
  if (a.write_logits) a.logits = route->logits;
  if (persistent) {
    // two launches: router (+ shared work items, hand-off words cleared), then
    // one persistent kernel for top-k, buckets, gate/up, down and combine; the
    // route copies of the layer input go first (a stack's combine overwrites it)
    if (route && (e = copy_async(route->x_in, a.x, (size_t)a.T * moe::D_MODEL * 2, s)) != hipSuccess)
      return hip_fail(e, "route copy");
    if ((e = moe::launch_decode(a, reinterpret_cast<uint32_t*>(ws + W.sync), L->n_cu, s)) != hipSuccess)
      return hip_fail(e, "persistent decode launch");
    if (route) {
      const size_t S = (size_t)a.S;
      const int E = a.E;
      if ((e = copy_async(route->topk_ids, a.ids, S * 4, s)) != hipSuccess ||
          (e = copy_async(route->topk_w, a.w, S * 4, s)) != hipSuccess ||
          (e = copy_async(route->counts, a.counts, (size_t)E * 4, s)) != hipSuccess ||
          (e = copy_async(route->offsets, a.offsets, (size_t)(E + 1) * 4, s)) != hipSuccess ||
          (e = copy_async(route->perm, a.perm, S * 4, s)) != hipSuccess ||
          (e = copy_async(route->inv_perm, a.inv_perm, S * 4, s)) != hipSuccess)
        return hip_fail(e, "route copy");
    }
    return MOE_OK;
  }
  if ((e = mark(ev, 0, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_router(a, s)) != hipSuccess) return hip_fail(e, "router launch");
  if ((e = mark(ev, 1, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_topk(a, s)) != hipSuccess) return hip_fail(e, "top-k launch");
  if ((e = mark(ev, 2, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_bucket(a, s)) != hipSuccess) return hip_fail(e, "bucket launch");
  if (route) {
    const size_t S = (size_t)a.S;
    const int E = a.E;
    if ((e = copy_async(route->topk_ids, a.ids, S * 4, s)) != hipSuccess ||
        (e = copy_async(route->topk_w, a.w, S * 4, s)) != hipSuccess ||
        (e = copy_async(route->counts, a.counts, (size_t)E * 4, s)) != hipSuccess ||
        (e = copy_async(route->offsets, a.offsets, (size_t)(E + 1) * 4, s)) != hipSuccess ||
        (e = copy_async(route->perm, a.perm, S * 4, s)) != hipSuccess ||
        (e = copy_async(route->inv_perm, a.inv_perm, S * 4, s)) != hipSuccess ||
        (e = copy_async(route->x_in, a.x, (size_t)a.T * moe::D_MODEL * 2, s)) != hipSuccess)
      return hip_fail(e, "route copy");
  }
  if ((e = mark(ev, 3, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_ffn(a, true, L->n_cu, W.max_tiles * moe::vec_up_chunks(a.T), s)) != hipSuccess)
    return hip_fail(e, "gate/up launch");
  if ((e = mark(ev, 4, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_ffn(a, false, L->n_cu, W.max_tiles * moe::vec_dn_chunks(a.T), s)) != hipSuccess)
    return hip_fail(e, "down launch");
  if ((e = mark(ev, 5, s)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = moe::launch_combine(a, s)) != hipSuccess) return hip_fail(e, "combine launch");
  if ((e = mark(ev, 6, s)) != hipSuccess) return hip_fail(e, "event record");
  return MOE_OK;
}

moe_status check_ws(void* ws, size_t have, size_t need) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return MOE_OK;
}

// Decode attention: positions per split and the split count for B sequences of
// at most max_len positions (the splits cover the attended span and the
// alignment of its start down to 64); smaller splits while there would be
// fewer than 1024 waves.
struct AttnPlan {
  int splits;
  size_t q_off, o_off, ml_off, total;
};
moe_status attn_plan(const moe_attn_desc* d, int32_t B, int32_t max_len, AttnPlan* P) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "attention descriptor is NULL");
  if (d->window < 0) return fail(MOE_ERR_INVALID_ARG, "window=%d must be >= 0", d->window);
  if (d->rope != 0 && d->rope != 1) return fail(MOE_ERR_INVALID_ARG, "rope=%d must be 0 or 1", d->rope);
  if (d->rope && !(d->rope_theta > 0.f)) return fail(MOE_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (!(d->rms_eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if (B < 0 || B > 65535) return fail(MOE_ERR_INVALID_ARG, "B=%d outside [0, 65535]", B);
  if (max_len < 1) return fail(MOE_ERR_INVALID_ARG, "max_len=%d must be >= 1", max_len);
  // about 512 / (4 B) splits of 4 waves, so that the workgroups fill the GPU
  // about once and each wave streams several 32-position steps; at most 64, and
  // no more than there are groups of 4 steps in the attended span.  Spans of up
  // to 1024 positions (the 513-token window among them) take one split: each
  // wave then has at most 8 steps, and no combine kernel runs.
  const int span = (d->window > 0 && d->window < max_len ? d->window : max_len) + 63;
  const int groups = (span + 32 * 4 - 1) / (32 * 4);
  P->splits = span <= 1024 + 63 ? 1 : std::min({std::max(1, (512 + 4 * B - 1) / (4 * std::max(B, 1))), 64, groups});
  const size_t rows = (size_t)B * moe::ATTN_HQ;
  P->q_off = 0;
  P->o_off = up256(rows * moe::ATTN_D * 2);
  P->ml_off = P->o_off + up256(rows * P->splits * moe::ATTN_D * 4);
  P->total = P->ml_off + up256(rows * P->splits * 2 * 4);
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* w, moe_layer** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (!w->router_w || !aligned(w->router_w, 16))
    return fail(MOE_ERR_INVALID_ARG, "router_w is NULL or not 16-byte aligned");
  if (w->router_b && !aligned(w->router_b, 4)) return fail(MOE_ERR_INVALID_ARG, "router_b is not 4-byte aligned");
  const int f = desc->wfmt;
  if ((st = check_qmat(w->gate, f, "gate")) || (st = check_qmat(w->up, f, "up")) ||
      (st = check_qmat(w->down, f, "down")))
    return st;
  if (desc->n_shared && ((st = check_qmat(w->sh_gate, f, "sh_gate")) || (st = check_qmat(w->sh_up, f, "sh_up")) ||
                         (st = check_qmat(w->sh_down, f, "sh_down"))))
    return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev, prop.gcnArchName);
  moe_layer* L = new (std::nothrow) moe_layer;
  if (!L) return fail(MOE_ERR_INVALID_ARG, "out of host memory");
  L->desc = *desc;
  L->w = *w;
  L->device = dev;
  L->n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  *out = L;
  return MOE_OK;
}

void moe_layer_destroy(moe_layer* layer) { delete layer; }

moe_status moe_desc_workspace_size(const moe_layer_desc* desc, int32_t T, size_t* bytes) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  if (T < 0 || T > desc->max_tokens) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, max_tokens=%d]", T, desc->max_tokens);
  *bytes = ws_layout(*desc, T).total;
  return MOE_OK;
}

moe_status moe_layer_workspace_size(const moe_layer* layer, int32_t T, size_t* bytes) {
  if (!layer) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  return moe_desc_workspace_size(&layer->desc, T, bytes);
}

static moe_status layer_forward_impl(const moe_layer* L, const void* x, int32_t T, void* y,
                                     const moe_route_out* route, void* ws, size_t ws_bytes, void* stream,
                                     void* const* ev, bool persistent = false) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (T < 0 || T > L->desc.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, max_tokens=%d]", T, L->desc.max_tokens);
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
  if (!y || !aligned(y, 16)) return fail(MOE_ERR_INVALID_ARG, "y is NULL or not 16-byte aligned");
  const size_t xb = (size_t)T * moe::D_MODEL * 2;
  if ((const char*)x < (const char*)y + xb && (const char*)y < (const char*)x + xb)
    return fail(MOE_ERR_INVALID_ARG, "x and y overlap");
  const WsLayout W = ws_layout(L->desc, T);
  moe_status st = check_ws(ws, ws_bytes, W.total);
  if (st != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (persistent && !moe::decode_supported(T))
    return fail(MOE_ERR_UNSUPPORTED, "the persistent decode path covers 1..64 tokens (T=%d)", T);
  moe::LayerArgs a = make_args(L, x, T, (char*)ws, W);
  a.out = (uint16_t*)y;
  if ((st = run_layer(L, a, W, route, s, ev, (char*)ws, persistent)) != MOE_OK) return st;
  hipError_t e;
  if (route && (e = copy_async(route->y_out, y, xb, s)) != hipSuccess) return hip_fail(e, "route copy");
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer* L, const void* x, int32_t T, void* y, const moe_route_out* route,
                             void* ws, size_t ws_bytes, void* stream) {
  return layer_forward_impl(L, x, T, y, route, ws, ws_bytes, stream, nullptr);
}

// Workspace of moe_layer_forward_noalloc: one copy per GPU, held by the loaded
// code object until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels and copies get the device address
// that hipGetSymbolAddress returns for the current device (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_MAX_WORKSPACE];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once taken

// The device address of `scratch` on device dev, which must be current.
moe_status scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

moe_status moe_layer_forward_noalloc(const moe_layer* L, const void* x, int32_t T, void* y,
                                     const moe_route_out* route, void* stream) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "layer is NULL");
  if (T < 0 || T > L->desc.max_tokens)
    return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, max_tokens=%d]", T, L->desc.max_tokens);
  if (T == 0) return MOE_OK;
  const size_t need = ws_layout(L->desc, T).total;
  if (need > (size_t)MOE_NOALLOC_MAX_WORKSPACE)
    return fail(MOE_ERR_WORKSPACE, "T=%d needs %zu workspace bytes; the static scratch holds %zu", T, need,
                (size_t)MOE_NOALLOC_MAX_WORKSPACE);
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != L->device)
    return fail(MOE_ERR_INVALID_ARG, "device %d is current; the layer was created on device %d", dev, L->device);
  void* ws = nullptr;
  const moe_status st = scratch_ptr(dev, &ws);
  if (st != MOE_OK) return st;
  return layer_forward_impl(L, x, T, y, route, ws, (size_t)MOE_NOALLOC_MAX_WORKSPACE, stream, nullptr);
}

moe_status moe_layer_forward_persistent(const moe_layer* L, const void* x, int32_t T, void* y,
                                        const moe_route_out* route, void* ws, size_t ws_bytes, void* stream) {
  return layer_forward_impl(L, x, T, y, route, ws, ws_bytes, stream, nullptr, true);
}

moe_status moe_layer_forward_staged(const moe_layer* L, const void* x, int32_t T, void* y,
                                    const moe_route_out* route, void* ws, size_t ws_bytes, void* stream,
                                    void* const* events, int32_t n_events) {
  if (!events || n_events != MOE_N_STAGE_EVENTS)
    return fail(MOE_ERR_INVALID_ARG, "events must hold %d hipEvent_t", MOE_N_STAGE_EVENTS);
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "events[%d] is NULL", i);
  return layer_forward_impl(L, x, T, y, route, ws, ws_bytes, stream, events);
}

moe_status moe_stack_workspace_size(const moe_layer* const* layers, int32_t n, int32_t T, size_t* bytes) {
  if (!layers || n < 1) return fail(MOE_ERR_INVALID_ARG, "layers is NULL or n_layers < 1");
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  size_t mx = 0;
  for (int l = 0; l < n; ++l) {
    if (!layers[l]) return fail(MOE_ERR_INVALID_ARG, "layers[%d] is NULL", l);
    if (T < 0 || T > layers[l]->desc.max_tokens)
      return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, max_tokens] of layer %d", T, l);
    const size_t b = ws_layout(layers[l]->desc, T).total;
    if (b > mx) mx = b;
  }
  *bytes = mx + up256(sizeof(float) * (size_t)T * moe::D_MODEL) + up256(2 * (size_t)T * moe::D_MODEL);
  return MOE_OK;
}

static moe_status stack_forward_impl(const moe_layer* const* layers, int32_t n, void* x, int32_t T, float eps,
                                     const moe_route_out* routes, void* ws, size_t ws_bytes, void* stream,
                                     bool persistent) {
  size_t need = 0;
  moe_status st = moe_stack_workspace_size(layers, n, T, &need);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (persistent && !moe::decode_supported(T))
    return fail(MOE_ERR_UNSUPPORTED, "the persistent decode path covers 1..64 tokens (T=%d)", T);
  if (!x || !aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
  if (!(eps >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "rms_eps must be >= 0");
  if ((st = check_ws(ws, ws_bytes, need)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  size_t layer_ws = 0;
  for (int l = 0; l < n; ++l) {
    const size_t b = ws_layout(layers[l]->desc, T).total;
    if (b > layer_ws) layer_ws = b;
  }
  char* base = (char*)ws;
  float* r = (float*)(base + layer_ws);
  uint16_t* xn = (uint16_t*)(base + layer_ws + up256(sizeof(float) * (size_t)T * moe::D_MODEL));
  hipError_t e = moe::launch_stack_init((const uint16_t*)x, r, xn, T, eps, s);
  if (e != hipSuccess) return hip_fail(e, "stack init launch");
  for (int l = 0; l < n; ++l) {
    const moe_layer* L = layers[l];
    const WsLayout W = ws_layout(L->desc, T);
    moe::LayerArgs a = make_args(L, xn, T, base, W);
    const moe_route_out* route = routes ? &routes[l] : nullptr;
    const bool last = (l == n - 1);
    a.r = r;
    a.eps = eps;
    a.y_rec = route ? (uint16_t*)route->y_out : nullptr;
    a.xn_next = last ? nullptr : xn;
    a.x_final = last ? (uint16_t*)x : nullptr;
    if ((st = run_layer(L, a, W, route, s, nullptr, base, persistent)) != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_stack_forward(const moe_layer* const* layers, int32_t n, void* x, int32_t T, float eps,
                             const moe_route_out* routes, void* ws, size_t ws_bytes, void* stream) {
  return stack_forward_impl(layers, n, x, T, eps, routes, ws, ws_bytes, stream, false);
}

moe_status moe_stack_forward_persistent(const moe_layer* const* layers, int32_t n, void* x, int32_t T, float eps,
                                        const moe_route_out* routes, void* ws, size_t ws_bytes, void* stream) {
  return stack_forward_impl(layers, n, x, T, eps, routes, ws, ws_bytes, stream, true);
}

moe_status moe_head_forward(const void* x, int32_t T, const moe_qmat* w, int32_t wfmt, int32_t vocab,
                            int32_t d_model, float* logits, void* stream) {
  if (T < 0 || T > 65536) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 65536]", T);
  if (vocab < 1 || vocab > MOE_HEAD_MAX_VOCAB)
    return fail(MOE_ERR_INVALID_ARG, "vocab=%d outside [1, %d]", vocab, MOE_HEAD_MAX_VOCAB);
  if (wfmt < MOE_W_BF16 || wfmt > MOE_W_NVFP4) return fail(MOE_ERR_INVALID_ARG, "unknown wfmt %d", wfmt);
  if (d_model != moe::D_MODEL)
    return fail(MOE_ERR_UNSUPPORTED, "this build has head kernels for d_model=%d (got %d)", moe::D_MODEL, d_model);
  if (!w) return fail(MOE_ERR_INVALID_ARG, "w is NULL");
  moe_status st = check_qmat(*w, wfmt, "head");
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
  if (!logits || !aligned(logits, 4)) return fail(MOE_ERR_INVALID_ARG, "logits is NULL or not 4-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int n_cu = 0;
  if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return hip_fail(e, "device query");
  moe::HeadArgs a;
  a.x = (const uint16_t*)x;
  a.w = qm(*w);
  a.logits = logits;
  a.T = T;
  a.V = vocab;
  a.fmt = wfmt;
  if ((e = moe::launch_head(a, n_cu > 0 ? n_cu : 256, (hipStream_t)stream)) != hipSuccess)
    return hip_fail(e, "head launch");
  return MOE_OK;
}

moe_status moe_stream_read(const void* src, size_t bytes, void* sink, int32_t grid, void* stream) {
  if (!src || !aligned(src, 16)) return fail(MOE_ERR_INVALID_ARG, "src must be a 16 B aligned device pointer");
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (!sink || !aligned(sink, 4)) return fail(MOE_ERR_INVALID_ARG, "sink must be a 4 B aligned device pointer");
  if (grid < 0 || grid > 65536) return fail(MOE_ERR_INVALID_ARG, "grid must be in [0, 65536], got %d", grid);
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  if ((e = moe::launch_stream_read(src, bytes, static_cast<uint32_t*>(sink), grid ? grid : n_cu,
                                   static_cast<hipStream_t>(stream))) != hipSuccess)
    return hip_fail(e, "stream read launch");
  return MOE_OK;
}

moe_status moe_mfma_rate(int32_t kind, int32_t iters, int32_t grid, float* sink, void* stream) {
  if (kind < 0 || kind > 3) return fail(MOE_ERR_INVALID_ARG, "kind must be 0..3, got %d", kind);
  if (iters < 1 || iters > (1 << 24)) return fail(MOE_ERR_INVALID_ARG, "iters must be in [1, 2^24], got %d", iters);
  if (grid < 1 || grid > 65536) return fail(MOE_ERR_INVALID_ARG, "grid must be in [1, 65536], got %d", grid);
  if (!sink || !aligned(sink, 4)) return fail(MOE_ERR_INVALID_ARG, "sink must be a 4 B aligned device pointer");
  const hipError_t e = moe::launch_mfma_rate(kind, iters, grid, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "matrix-core rate launch");
  return MOE_OK;
}

moe_status moe_read_pattern(int32_t pattern, const void* src, size_t bytes, size_t row_bytes, int32_t grid,
                            void* sink, void* stream) {
  if (!moe::read_pattern_shape_ok(pattern, bytes, row_bytes))
    return fail(MOE_ERR_INVALID_ARG,
                "pattern must be 0..4, row_bytes a positive multiple of 256, and bytes a positive multiple of the "
                "pattern's rows (32, 32, 32, 4, 8) times row_bytes (pattern %d, bytes %zu, row_bytes %zu)",
                pattern, bytes, row_bytes);
  if (!src || !aligned(src, 16)) return fail(MOE_ERR_INVALID_ARG, "src must be a 16 B aligned device pointer");
  if (!sink || !aligned(sink, 4)) return fail(MOE_ERR_INVALID_ARG, "sink must be a 4 B aligned device pointer");
  if (grid < 1 || grid > 65536) return fail(MOE_ERR_INVALID_ARG, "grid must be in [1, 65536], got %d", grid);
  const hipError_t e = moe::launch_read_pattern(pattern, src, bytes, row_bytes, grid, static_cast<uint32_t*>(sink),
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "read-pattern launch");
  return MOE_OK;
}

moe_status moe_release_cost(int32_t mode, float* data, uint32_t* counters, int32_t grid, int32_t per_thread,
                            void* stream) {
  if (mode < 0 || mode > 4) return fail(MOE_ERR_INVALID_ARG, "mode must be 0..4, got %d", mode);
  if (grid < 1 || grid > 65536) return fail(MOE_ERR_INVALID_ARG, "grid must be in [1, 65536], got %d", grid);
  if (per_thread < 1 || per_thread > 64)
    return fail(MOE_ERR_INVALID_ARG, "per_thread must be in [1, 64], got %d", per_thread);
  if (!data || !aligned(data, 4)) return fail(MOE_ERR_INVALID_ARG, "data must be a 4 B aligned device pointer");
  if (!counters || !aligned(counters, 4)) return fail(MOE_ERR_INVALID_ARG, "counters must be a 4 B aligned device pointer");
  const hipError_t e = moe::launch_release_cost(mode, data, counters, grid, per_thread, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "release-cost launch");
  return MOE_OK;
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe_ffn gfx950 0.1"; }

}  // extern "C"

moe_status moe_attn_workspace_size(const moe_attn_desc* d, int32_t B, int32_t max_len, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  AttnPlan P;
  moe_status st = attn_plan(d, B, max_len, &P);
  if (st != MOE_OK) return st;
  *bytes = P.total;
  return MOE_OK;
}

moe_status moe_attn_decode(const moe_attn_desc* d, int32_t B, int32_t max_len, const void* q, const void* k,
                           const void* v, const void* q_gain, const void* k_gain, const float* sinks,
                           const int32_t* pos, void* k_cache, void* v_cache_t, int32_t cap, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  AttnPlan P;
  moe_status st = attn_plan(d, B, max_len, &P);
  if (st != MOE_OK) return st;
  if (cap < 64 || cap % 64) return fail(MOE_ERR_INVALID_ARG, "cap=%d must be a positive multiple of 64", cap);
  if (max_len > cap) return fail(MOE_ERR_INVALID_ARG, "max_len=%d exceeds cap=%d", max_len, cap);
  if (B == 0) return MOE_OK;
  struct { const void* p; size_t al; const char* name; } ptrs[] = {
      {q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"}, {q_gain, 2, "q_gain"}, {k_gain, 2, "k_gain"}, {pos, 4, "pos"},
      {k_cache, 16, "k_cache"}, {v_cache_t, 16, "v_cache_t"}, {out, 4, "out"}, {workspace, 256, "workspace"}};
  for (const auto& e : ptrs)
    if (!e.p || !aligned(e.p, e.al)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL or not %zu-byte aligned", e.name, e.al);
  if (sinks && !aligned(sinks, 4)) return fail(MOE_ERR_INVALID_ARG, "sinks is not 4-byte aligned");
  if (workspace_bytes < P.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, P.total);
  moe::AttnArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.q_gain = (const uint16_t*)q_gain;
  a.k_gain = (const uint16_t*)k_gain;
  a.sinks = sinks;
  a.pos = pos;
  a.k_cache = (uint16_t*)k_cache;
  a.v_cache = (uint16_t*)v_cache_t;
  char* ws = (char*)workspace;
  a.qbuf = (uint16_t*)(ws + P.q_off);
  a.part_o = (float*)(ws + P.o_off);
  a.part_ml = (float*)(ws + P.ml_off);
  a.out = (uint16_t*)out;
  a.cap = cap;
  a.window = d->window;
  a.rope = d->rope;
  a.splits = P.splits;
  a.eps = d->rms_eps;
  const double th = d->rope ? (double)d->rope_theta : 1.0;
  for (int e = 0; e < 8; ++e) a.rot_e[e] = pow(th, -2.0 * e / moe::ATTN_D);
  for (int g = 0; g < 4; ++g) a.rot_g[g] = pow(th, -2.0 * 8 * g / moe::ATTN_D);
  a.rot_32 = pow(th, -2.0 * 32 / moe::ATTN_D);
  hipError_t e = moe::launch_attn(a, B, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MOE_OK;
}
