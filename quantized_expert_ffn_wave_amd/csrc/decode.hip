// Persistent decode layer: the whole MoE layer forward of a decode batch (no
// bucket or shared expert large enough for matrix-core tiles, i.e. up to 64
// tokens) in two launches instead of five or six.
//
// The review "Recursive Flint 40B-A2.5B", section "The quantisation recipe is
// the most transferable part", describes a kernel that fuses the whole decode
// pass into one dispatch on its laptop hardware.  On gfx950 the same idea
// meets eight XCDs with separate L2 caches: a hand-off between workgroups on
// different XCDs needs an agent-scope release (write-back of the XCD's L2) and
// acquire (invalidation), which is what a kernel boundary does too.  So this
// path keeps the one boundary that is free of ordering cost and turns the rest
// into in-kernel hand-offs:
//   launch A  the router's partial logits (as router_small_kernel), and in its
//             first workgroup the shared expert's work items (they do not
//             depend on the routing) and the hand-off counters cleared;
//   launch B  persistent, one workgroup per CU (all resident at once):
//     1. top-k, a wave per token, on the first ceil(T/4) workgroups; each
//        publishes its ids and counts itself in, and the last one to arrive
//        builds the buckets and work lists.  Meanwhile the other workgroups
//        run the shared expert's gate/up items;
//     2. grid barrier, then the routed gate/up items;
//     3. grid barrier, then every down item (routed and shared);
//     4. grid barrier, then the combine, a workgroup per token (with the
//        residual and RMSNorm glue in a stack).
// A hand-off: every wave waits for its own stores, the workgroup meets at a
// barrier, and its first thread issues an agent-scope release and adds itself
// to a counter; the waiters spin on the counter with agent-scope loads (a
// bounded spin: past it the workgroup goes on and marks the timeout word) and
// then issue an agent-scope acquire.  All workgroups are resident, so every
// wait ends.
#include "common.hpp"

namespace moe {

constexpr int DEC_MAX_T = 64;  // largest batch with no matrix-core tile at all
static_assert(!bucket_mfma(DEC_MAX_T, DEC_MAX_T) && !shared_mfma(DEC_MAX_T) && shared_mfma(DEC_MAX_T + 1),
              "the persistent path covers exactly the batches without matrix-core tiles");
constexpr int DEC_SPIN_LIMIT = 1 << 18;  // polls of about 1 us: a wait gives up after about 0.3 s

// This wave's stores are complete, then the workgroup meets: afterwards one
// thread's agent-scope release covers the whole workgroup's stores.
__device__ inline void wg_drain() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// The workgroup counts itself into ctr (n arrivals expected); true in every
// thread of the last workgroup to arrive, after its acquire.
__device__ inline bool last_arrival(uint32_t* ctr, uint32_t n) {
  __shared__ uint32_t last;
  wg_drain();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = (old == n - 1) ? 1u : 0u;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return last != 0u;
}

// All n workgroups meet at counter ctr.
__device__ inline void grid_barrier(uint32_t* ctr, uint32_t n, uint32_t* timeout) {
  wg_drain();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n && spins < DEC_SPIN_LIMIT) {
      __builtin_amdgcn_s_sleep(1);
      ++spins;
    }
    if (spins >= DEC_SPIN_LIMIT) __hip_atomic_store(timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void decode_router_kernel(LayerArgs a, uint32_t* sync) {
  router_small_tile(a.x, a.router_w, a.router_b, a.logit_part, a.T, a.E, blockIdx.x, blockIdx.y);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    const int tid = threadIdx.x;
    if (tid < DEC_SYNC_WORDS) sync[tid] = 0u;
    const int sh = a.n_shared ? shared_tiles(a.T) : 0;  // vector tiles at the front of the list
    for (int i = tid; i < sh; i += blockDim.x) a.tiles[i] = shared_tile(a.T, i, false, 0);
  }
}

template <int FMT, int VR, int VDR>
__global__ __launch_bounds__(256, (FFN_WG_PER_CU<FMT, 0>)) void decode_layer_kernel(LayerArgs a, uint32_t* sync) {
  __shared__ union {
    MvSmem gv;
    RouteSmallSmem rs;
  } sm;
  const int G = (int)gridDim.x, w = (int)blockIdx.x, wave = (int)threadIdx.x >> 6;
  const int n_tk = ceil_div(a.T, 4);  // top-k workgroups, a wave per token
  const int n_sh = (a.n_shared ? shared_tiles(a.T) : 0) * (D_FF / VR);  // shared gate/up items (list front)
  uint32_t* timeout = sync + DEC_SYNC_TIMEOUT;
  if (w < n_tk) {
    const int t = 4 * w + wave;
    if (t < a.T) topk_token<ROUTER_KS>(a, t, nullptr);
    if (last_arrival(sync + DEC_SYNC_TOPK, (uint32_t)n_tk)) route_small<false>(a, sm.rs);
  } else if (n_sh > 0) {
    up_stream<FMT, VR>(a, 0, n_sh, 0, sm.gv, w - n_tk, G - n_tk);
  }
  grid_barrier(sync + DEC_SYNC_B1, (uint32_t)G, timeout);
  // (the counts come from another workgroup in this launch: agent-scope loads)
  const int n_up = (int)__hip_atomic_load(a.ctl + CTL_N_UP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n_dn = (int)__hip_atomic_load(a.ctl + CTL_N_DN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  up_stream<FMT, VR>(a, n_sh, n_up - n_sh, 0, sm.gv, w, G);
  grid_barrier(sync + DEC_SYNC_B2, (uint32_t)G, timeout);
  down_stream<FMT, VDR>(a, 0, n_dn, 0, sm.gv, w, G);
  grid_barrier(sync + DEC_SYNC_B3, (uint32_t)G, timeout);
  for (int t = w; t < a.T; t += G) combine_token(a, t);
}

template <int FMT, int VR, int VDR>
hipError_t launch_decode_var(const LayerArgs& a, uint32_t* sync, int n_cu, hipStream_t s) {
  // One workgroup per CU (the kernel fits two or three): every workgroup is
  // resident at once, so every wait ends.  Each hand-off costs every workgroup
  // an L2 write-back and invalidation; measured on the 4-token layer, 768
  // workgroups took 206 us per forward and 256 took 63 us (the kernel chain: 31).
  const int grid = n_cu;
  hipLaunchKernelGGL(decode_router_kernel, dim3(ceil_div(a.T, 16) * ceil_div(a.E, 64), ROUTER_KS), dim3(256), 0, s,
                     a, sync);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_layer_kernel<FMT, VR, VDR>), dim3(grid), dim3(256), 0, s, a, sync);
  return hipGetLastError();
}

template <int FMT> hipError_t launch_decode_fmt(const LayerArgs& a, uint32_t* sync, int n_cu, hipStream_t s) {
  if (a.T <= 1) return launch_decode_var<FMT, 16, 128>(a, sync, n_cu, s);
  if (a.T <= VEC_SMALL_T) return launch_decode_var<FMT, 32, 128>(a, sync, n_cu, s);
  return launch_decode_var<FMT, UP_ROWS, DN_ROWS>(a, sync, n_cu, s);
}

bool decode_supported(int T) { return T >= 1 && T <= DEC_MAX_T; }

hipError_t launch_decode(const LayerArgs& a, uint32_t* sync, int n_cu, hipStream_t s) {
  switch (a.fmt) {
    case FMT_Q4_1: return launch_decode_fmt<FMT_Q4_1>(a, sync, n_cu, s);
    case FMT_NVFP4: return launch_decode_fmt<FMT_NVFP4>(a, sync, n_cu, s);
    default: return launch_decode_fmt<FMT_BF16>(a, sync, n_cu, s);
  }
}

}  // namespace moe
