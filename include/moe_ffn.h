/*
 * moe_ffn.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts layer.
 *
 * The operation is the MoE layer of the open-weight coding model reviewed on
 * orcarouter.ai as "Recursive Flint 40B-A2.5B", section "The architecture is
 * an argument about memory bandwidth": per MoE layer, 256 routed experts of
 * which each token uses 6, plus one shared expert that every token uses, with
 * 47 such layers in the model; the same section states that decoding is bound
 * by moving weights from memory.  The 4-bit storage formats (q4_1 and NVFP4)
 * and the 16-bit checkpoint are the artefacts listed in "What actually
 * shipped".  The page does not give the expert width, the activation or the
 * router form; this library computes, per token x (bf16, d_model wide):
 *
 *   logits = x Wr^T + b                     (bf16 operands, fp32 accumulate)
 *   ids    = the top_k largest logits, ties to the lower expert id
 *   w      = softmax over the chosen logits (renorm_topk = 1), or the chosen
 *            entries of the softmax over all experts (renorm_topk = 0)
 *   E_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x))  (SwiGLU, silu(g) = g/(1+e^-g))
 *   y      = sum_j w_j E_{ids_j}(x) + shared_scale * E_shared(x)   -> bf16
 *
 * Arithmetic: router logits accumulate in fp32 from bf16 operands; expert
 * outputs are summed in fp32 in the order j = 0..k-1, then the shared expert,
 * and the result is rounded once to bf16.  With bf16 weights both expert
 * products run on bf16 operands, the SwiGLU output h is rounded to bf16
 * between them, and each expert output is rounded to bf16 (RNE) before the
 * sum.  With 4-bit weights both expert products run on fp16 operands (every
 * q4_1 weight d*q + m rounded once to fp16, every NVFP4 E2M1 x E4M3 product
 * exact in fp16, the tensor scale applied in fp32), h and the expert outputs
 * stay fp32, and each token's activations (x, and h per expert-output row)
 * enter the products multiplied by a power of two that puts the row's largest
 * magnitude in [2^14, 2^15), undone in fp32 afterwards: the size of a token
 * row is then limited only by fp32, not by fp16's range.
 * Supported inputs: finite x (NaN and infinity are outside the contract);
 * finite weights with every q4_1 block satisfying |d*q + m| <= 65504 for
 * q = 0..15; results whose intermediate values (logits, gate/up products, h,
 * expert outputs) are finite in fp32.  The library does not check these.
 *
 * and moe_stack_forward chains layers as a pre-norm residual stack:
 *   r <- x;  for each layer: r <- r + bf16(layer(bf16(RMSNorm(r))));  x <- bf16(r)
 * with RMSNorm(r) = r / sqrt(mean(r^2) + eps) (gain 1) and r kept in fp32.
 *
 * Conventions for every call:
 *   - returns a moe_status; never aborts or throws; moe_last_error() gives a
 *     thread-local message for the last non-OK status of the calling thread;
 *   - every argument is checked on the host before any work is enqueued;
 *   - all device memory (weights, activations, workspace, route outputs) is
 *     owned by the caller; the library never allocates device memory, and the
 *     weight arrays are borrowed by a layer handle and must outlive it;
 *   - forward calls are asynchronous on the given HIP stream (a hipStream_t
 *     passed as void*, NULL = the default stream); MOE_OK means enqueued, the
 *     results are valid once the caller synchronises that stream; no call
 *     synchronises the host and data-dependent sizes stay on the device, so a
 *     forward can be captured in a HIP graph;
 *   - a layer handle is immutable after create and holds no GPU resources;
 *     every forward runs as one chain of kernels on the caller's stream (the
 *     shared expert's work sits in the same work lists as the routed
 *     experts'); concurrent forwards on one handle are safe when each uses
 *     its own workspace and outputs.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a NULL/misaligned pointer, a bad size or shape, T > max_tokens */
  MOE_ERR_UNSUPPORTED = 2, /* not a gfx950 device, or a shape/format this build has no kernels for */
  MOE_ERR_WORKSPACE = 3,   /* workspace NULL, misaligned (256 B) or smaller than the size query returns */
  MOE_ERR_HIP = 4          /* a HIP runtime call failed (no device, launch failure); message has its name */
} moe_status;

/* Storage format of the expert weights (routed and shared alike). */
typedef enum {
  MOE_W_BF16 = 0,  /* plain bf16, the 16-bit checkpoint ("What actually shipped", BF16 bullet) */
  MOE_W_Q4_1 = 1,  /* q4_1 ("What actually shipped", Int4 GGUF bullet): blocks of 32 along a row,
                      w = d*q + m, q unsigned 4-bit, d and m fp16 */
  MOE_W_NVFP4 = 2  /* NVFP4 ("What actually shipped", NVFP4 GGUF bullet): blocks of 16 along a row,
                      w = E2M1(c) * E4M3(s) * ts, one OCP E4M3FN scale s per block, fp32 ts per matrix */
} moe_wfmt;

/* Shape and options of one MoE layer.  This build has kernels for
 * d_model = 2048 and d_expert = d_shared = 512 (the reviewed model's MoE
 * layer shape); other widths return MOE_ERR_UNSUPPORTED. */
typedef struct {
  int32_t d_model;      /* hidden size: 2048 */
  int32_t n_experts;    /* routed experts: multiple of 16, 16..256 (the model: 256) */
  int32_t top_k;        /* experts chosen per token: 1..8, <= n_experts (the model: 6) */
  int32_t d_expert;     /* routed expert width: 512 */
  int32_t n_shared;     /* always-on shared experts: 0 or 1 (the model: 1) */
  int32_t d_shared;     /* shared expert width: must equal d_expert */
  float shared_scale;   /* weight of the shared expert's output (1.0) */
  int32_t renorm_topk;  /* 1: chosen weights sum to 1; 0: plain softmax entries */
  int32_t wfmt;         /* a moe_wfmt */
  int32_t max_tokens;   /* capacity: forwards accept 0 <= T <= max_tokens (1..65536) */
} moe_layer_desc;

/* One stored matrix set [n][rows][cols] (device pointers, row-major, the
 * reduction dimension `cols` contiguous).  Element 2i of a row is the LOW
 * nibble of byte i for the 4-bit formats.
 *   codes : q4_1 / NVFP4: uint8 [n][rows][cols/2]; bf16: bf16 [n][rows][cols]  (16 B aligned)
 *   scales: q4_1: fp16 pairs {d, m} [n][rows][cols/32][2]                      (16 B aligned)
 *           NVFP4: E4M3 bytes [n][rows][cols/16], a 32-element block's two     (8 B aligned)
 *                  scales adjacent (its first 16 elements' first)
 *           bf16: NULL
 *           Within a row of C = cols/32 blocks, block k's scales sit at block
 *           position (k mod 16) * (C/16) + floor(k/16) (C a multiple of 16;
 *           for cols = 512 that is the natural order), so that the 4 blocks
 *           k, k+16, k+32, k+48 of a row of 2048 are adjacent: the vector path
 *           reads them with one 16-byte (q4_1) or 8-byte (NVFP4) load.
 *   tensor_scale: NVFP4: fp32 [n]; otherwise NULL */
typedef struct {
  const void* codes;
  const void* scales;
  const float* tensor_scale;
} moe_qmat;

/* Weights of one layer (device pointers, borrowed by the handle). */
typedef struct {
  const void* router_w;   /* bf16 [n_experts][d_model] (16 B aligned) */
  const float* router_b;  /* fp32 [n_experts], or NULL for no router bias */
  moe_qmat gate, up;      /* routed: n = n_experts, rows = d_expert, cols = d_model */
  moe_qmat down;          /* routed: n = n_experts, rows = d_model, cols = d_expert */
  moe_qmat sh_gate, sh_up, sh_down; /* shared (n = 1, same shapes); ignored when n_shared = 0 */
} moe_layer_weights;

/* Optional copies of intermediate results (device pointers; each may be NULL).
 * T tokens, k = top_k, E = n_experts, S = T*k slots, slot s = t*k + j. */
typedef struct {
  int32_t* topk_ids; /* [T][k] chosen experts, logit-descending (ties: lower id first) */
  float* topk_w;     /* [T][k] routing weights, same order */
  float* logits;     /* [T][E] router logits (fp32, bias included) */
  int32_t* counts;   /* [E] slots per expert */
  int32_t* offsets;  /* [E+1] exclusive prefix sum of counts; offsets[E] = S */
  int32_t* perm;     /* [S] expert-sorted position -> slot; stable (token order inside a bucket) */
  void* x_in;        /* bf16 [T][d_model]: the layer's input (in a stack: bf16(RMSNorm(r))) */
  void* y_out;       /* bf16 [T][d_model]: the layer's output */
  int32_t* inv_perm; /* [S] slot -> its expert-sorted position (the inverse of perm) */
} moe_route_out;

typedef struct moe_layer moe_layer; /* opaque, host memory only */

/* Validate desc and weights (pointers, alignment), check that the current
 * device is gfx950, and return the handle.  No device memory is allocated and
 * no weight is repacked: the layouts above are the device layouts. */
moe_status moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* weights, moe_layer** out);

/* Free a handle (NULL-safe). */
void moe_layer_destroy(moe_layer* layer);

/* Workspace bytes a forward of T tokens needs (T <= max_tokens). */
moe_status moe_layer_workspace_size(const moe_layer* layer, int32_t T, size_t* bytes);

/* The same, from a descriptor alone (host-only; no device needed). */
moe_status moe_desc_workspace_size(const moe_layer_desc* desc, int32_t T, size_t* bytes);

/* One layer: y = MoE(x).  x, y: bf16 [T][d_model] device arrays (16 B aligned,
 * not overlapping).  route may be NULL.  workspace: device memory of at least
 * moe_layer_workspace_size bytes, 256 B aligned, used for this call only.
 * T = 0 is a no-op. */
moe_status moe_layer_forward(const moe_layer* layer, const void* x, int32_t T, void* y, const moe_route_out* route,
                             void* workspace, size_t workspace_bytes, void* stream);

/* moe_layer_forward that also records caller-created HIP events (hipEvent_t
 * passed as void*) on the caller's stream: events[i] just before stage i is
 * enqueued -- 0 router logits, 1 top-k, 2 buckets and work lists (for T <=
 * 16 built by stage 1's kernel, so stage 2 is empty), 3 gate/up + SwiGLU
 * (routed and shared experts), 4 down, 5 combine -- and events[6] after the
 * last stage.  n_events must be MOE_N_STAGE_EVENTS.  Used to time each
 * kernel on the stream it runs on; results are identical to
 * moe_layer_forward.  Event record failures return MOE_ERR_HIP. */
#define MOE_N_STAGE_EVENTS 7
moe_status moe_layer_forward_staged(const moe_layer* layer, const void* x, int32_t T, void* y,
                                    const moe_route_out* route, void* workspace, size_t workspace_bytes,
                                    void* stream, void* const* events, int32_t n_events);

/* moe_layer_forward without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a static array of MOE_NOALLOC_MAX_WORKSPACE bytes in the
 * library's code object, one copy per GPU, held until the process ends; its
 * address is taken once per device, on the first call with that device
 * current.  That bound covers every decode batch of up to 256 tokens of the
 * layers this build supports (moe_layer_workspace_size says what a forward
 * needs).
 *   layer, x, T, y, route, stream: as for moe_layer_forward; the layer's
 *            device must be current.
 * Errors: MOE_ERR_WORKSPACE when the forward of T tokens needs more than
 * MOE_NOALLOC_MAX_WORKSPACE bytes; MOE_ERR_INVALID_ARG for another current
 * device or the arguments moe_layer_forward rejects; MOE_ERR_HIP if the
 * scratch address cannot be taken.  All are returned before anything is
 * enqueued.  Every call on one GPU uses the same scratch and leaves its
 * contents there (nothing in it needs clearing: each forward writes what it
 * reads): calls whose execution overlaps on one GPU -- on two streams, or from
 * two threads -- race and give undefined results; order them on one stream. */
#define MOE_NOALLOC_MAX_WORKSPACE (32u << 20)
moe_status moe_layer_forward_noalloc(const moe_layer* layer, const void* x, int32_t T, void* y,
                                     const moe_route_out* route, void* stream);

/* moe_layer_forward as a persistent decode kernel, for batches of 1..64
 * tokens (those with no matrix-core tile): the review's section "The
 * quantisation recipe is the most transferable part" describes fusing the whole
 * decode pass into one dispatch.  Here it is two launches on the caller's
 * stream: the router (which also writes the shared expert's work items and
 * clears the hand-off words in the workspace), then one kernel with one
 * workgroup per compute unit (all resident at once) that runs top-k, buckets, gate/up,
 * down and the combine, handing results between its workgroups with
 * agent-scope release/acquire and counters in the workspace.  Results are
 * bit-identical to moe_layer_forward's.  Arguments, workspace size and errors
 * as for moe_layer_forward; T above 64 returns MOE_ERR_UNSUPPORTED.  Each
 * in-kernel wait is bounded: if the GPU cannot keep every workgroup of the
 * kernel resident (another kernel occupying compute units), the waits time out
 * and the outputs are undefined, so run it on an otherwise idle device or
 * stream order. */
moe_status moe_layer_forward_persistent(const moe_layer* layer, const void* x, int32_t T, void* y,
                                        const moe_route_out* route, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Workspace bytes for moe_stack_forward over these layers at T tokens. */
moe_status moe_stack_workspace_size(const moe_layer* const* layers, int32_t n_layers, int32_t T, size_t* bytes);

/* Pre-norm residual stack of n_layers layers (all with the same d_model and
 * format), updating x (bf16 [T][d_model]) in place.  routes: NULL or an array
 * of n_layers moe_route_out (each entry's pointers may be NULL). */
moe_status moe_stack_forward(const moe_layer* const* layers, int32_t n_layers, void* x, int32_t T, float rms_eps,
                             const moe_route_out* routes, void* workspace, size_t workspace_bytes, void* stream);

/* moe_stack_forward with every layer on the persistent decode path of
 * moe_layer_forward_persistent (two launches per layer; 1..64 tokens). */
moe_status moe_stack_forward_persistent(const moe_layer* const* layers, int32_t n_layers, void* x, int32_t T,
                                        float rms_eps, const moe_route_out* routes, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Output head (the step after the last MoE layer of a decode pass): logits
 * over the vocabulary,
 *   logits[t][v] = sum_k x[t][k] * W[v][k]      (fp32, K = d_model),
 * with W stored like an expert matrix (moe_qmat with n = 1, rows = vocab,
 * cols = d_model) in q4_1, NVFP4 or bf16.  The review's section "The
 * quantisation recipe is the most transferable part" stores this head in 4
 * bits because, with 2.5 B active parameters, it is a large share of the
 * weights each token reads; the vocabulary size is not given there.
 *   x      : bf16 [T][d_model] (16 B aligned), 0 <= T <= 65536
 *   logits : fp32 [T][vocab] (4 B aligned), written in full
 *   w, wfmt: the head matrix (device pointers, caller-owned, same alignment
 *            rules as the experts') and its format, MOE_W_BF16 / MOE_W_Q4_1 /
 *            MOE_W_NVFP4
 *   vocab  : 1 .. MOE_HEAD_MAX_VOCAB; d_model must be 2048 in this build
 * Asynchronous on `stream` like the layer forward; T = 0 is a no-op.  Bad
 * arguments return MOE_ERR_INVALID_ARG (MOE_ERR_UNSUPPORTED for d_model)
 * before anything is enqueued.  No workspace and no device allocation. */
#define MOE_HEAD_MAX_VOCAB 1048576
moe_status moe_head_forward(const void* x, int32_t T, const moe_qmat* w, int32_t wfmt, int32_t vocab,
                            int32_t d_model, float* logits, void* stream);

/* Measurement helper, not part of the layer: a plain streaming read of
 * `bytes` bytes of device memory at src, 16 bytes per load with eight loads in
 * flight per thread, on `grid` workgroups of 256 threads (0 = one per compute
 * unit) on the given stream.  It computes nothing and gives the attainable HBM
 * read rate that the layer's weight streams are measured against: the review's
 * section "The architecture is an argument about memory bandwidth" states that
 * decoding is bound by moving weights from memory.  src must be 16 B aligned
 * and bytes a positive multiple of 16; sink is caller-owned device memory of
 * 256 uint32 that the kernel may write (its contents are meaningless).
 * Invalid arguments return MOE_ERR_INVALID_ARG before anything is enqueued. */
moe_status moe_stream_read(const void* src, size_t bytes, void* sink, int32_t grid, void* stream);

/* Measurement helper, not part of the layer: grid workgroups of 256 threads
 * issue only matrix-core instructions of one kind, iters x 4 per wave in four
 * independent accumulator chains over operands held in registers:
 *   kind 0: v_mfma_f32_32x32x16_f16   (32768 flop each)
 *   kind 1: v_mfma_f32_32x32x16_bf16  (32768 flop each)
 *   kind 2: v_mfma_f32_32x32x16_fp8_fp8, E4M3 operands (32768 flop each)
 *   kind 3: v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 E2M1 operands and unit
 *           block scales (131072 flop each)
 * Timed by the caller, it gives the attainable rate of each kind, against which
 * the tile path's matrix-core utilisation is read; the FP4-class instruction is
 * the one the review's NVFP4 files ("What actually shipped") invite.  sink:
 * caller-owned device memory of 256 floats that the kernel overwrites (values
 * meaningless).  Bad arguments return MOE_ERR_INVALID_ARG before anything is
 * enqueued. */
moe_status moe_mfma_rate(int32_t kind, int32_t iters, int32_t grid, float* sink, void* stream);

/* Measurement helper, not part of the layer: the HBM read rate of one
 * per-instruction access pattern.  The review's section "The architecture is an
 * argument about memory bandwidth" makes the weight stream the bound; this
 * shows how the choice of bytes one load instruction touches moves that
 * stream.  The `bytes` bytes at src are split into regions of R rows of
 * row_bytes bytes, one region per wave at a time, each streamed with eight
 * 16-byte loads per lane in flight; a load instruction touches:
 *   pattern 0: 1 KB contiguous                  (R = 32)
 *   pattern 1: 32 rows x 32 bytes               (R = 32; per-lane operands of a 4-bit tile)
 *   pattern 2: 32 rows x 64 + 64 bytes          (R = 32; per-lane operands of a bf16 tile)
 *   pattern 3: 4 rows x 256 bytes               (R = 4; the vector path)
 *   pattern 4: 8 rows x 128 bytes               (R = 8; the tile loops' staged loads)
 * row_bytes: a positive multiple of 256; bytes: a positive multiple of
 * R x row_bytes; src 16 B aligned; grid workgroups of 256 threads; sink:
 * caller-owned device memory of 256 uint32 (contents meaningless).  Bad
 * arguments return MOE_ERR_INVALID_ARG before anything is enqueued. */
moe_status moe_read_pattern(int32_t pattern, const void* src, size_t bytes, size_t row_bytes, int32_t grid,
                            void* sink, void* stream);

/* Measurement helper, not part of the layer: the cost of the agent-scope
 * release that a hand-off between workgroups on different XCDs needs (the
 * alternative to a kernel boundary between the steps of the review's decode
 * pass, section "The quantisation recipe is the most transferable part").
 * grid workgroups of 256 threads each write per_thread floats per thread into
 * data (workgroup b owns floats [b * 256 * per_thread, (b + 1) * 256 *
 * per_thread)), then their first thread:
 *   mode 0: nothing more;  1: release fence + agent-scope atomic add of 1 to
 *   counters[16 (b mod 256)];  2: the atomic add only;  3: the release only;
 *   4: release, atomic add, acquire fence.
 * No workgroup waits for another.  data must hold grid * 256 * per_thread
 * floats and counters 4096 uint32 (caller-owned device memory; the counters are
 * incremented, not cleared).  grid in [1, 65536], per_thread in [1, 64]; bad
 * arguments return MOE_ERR_INVALID_ARG before anything is enqueued. */
moe_status moe_release_cost(int32_t mode, float* data, uint32_t* counters, int32_t grid, int32_t per_thread,
                            void* stream);

/* ---- decode attention ----------------------------------------------------------
 * One new token per sequence through one attention layer of the layout in the
 * review's section "The architecture is an argument about memory bandwidth":
 * 32 query heads share 4 key-value heads of dimension 128 (query head h reads
 * key-value head h / 8); sliding-window layers attend to the current token and
 * the 512 before it, the others to every earlier token; rotary position
 * embedding on the sliding-window layers only; an RMSNorm over each head of q
 * and k; a learned sink per query head.  Formulas (this library's reading):
 *   q' = bf16(rot(RMSNorm(q) * q_gain)), k' likewise with k_gain, where
 *   RMSNorm(x) = x / sqrt(mean(x^2) + rms_eps) over one head's 128 elements and
 *   rot pairs element i with i + 64 at angle pos * rope_theta^(-i/64);
 *   s_j = q'.k'_j / sqrt(128) over the attended positions j;
 *   out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink_h})   (bf16).
 * Cache layout (bf16, caller-owned device memory, cap positions per sequence,
 * cap a multiple of 64), one block of cap * 128 elements per (sequence b,
 * key-value head h) at offset (b * 4 + h) * cap * 128, laid out in the order the
 * matrix cores read it:
 *   k_cache   keys as stored (normalised and rotated): position p, dimension d
 *             at ((p / 16) * 16 + d / 8) * 128 + (p % 16) * 8 + d % 8
 *   v_cache_t values: position p = 32 a + 16 h + 4 g + s (h < 2, g < 4, s < 4),
 *             dimension d at (a * 8 + d / 16) * 512 + g * 128 + (d % 16) * 8 + 4 h + s
 * The call appends the new token's k' and v at position pos[b] and attends to
 * positions max(0, pos[b] + 1 - window) .. pos[b] (window 0: 0 .. pos[b]).
 * Entries the call does not attend to are never used, so an unwritten cache may
 * hold anything there. */
#define MOE_ATTN_Q_HEADS 32
#define MOE_ATTN_KV_HEADS 4
#define MOE_ATTN_HEAD_DIM 128
typedef struct {
  int32_t window;   /* 0: full attention; else the last `window` positions (513 on sliding-window layers) */
  int32_t rope;     /* 1: rotary embedding on q and k (sliding-window layers); 0: none */
  float rope_theta; /* base of the rotation frequencies, > 0 when rope is set (10000 in the benchmarks) */
  float rms_eps;    /* epsilon of the q/k RMSNorm, >= 0 (1e-6) */
} moe_attn_desc;

/* Workspace bytes for moe_attn_decode with B sequences of at most max_len
 * positions each (1 <= max_len <= cap; it sets the number of position splits). */
moe_status moe_attn_workspace_size(const moe_attn_desc* d, int32_t B, int32_t max_len, size_t* bytes);

/* The decode-attention step on `stream` (asynchronous, capturable): one
 * decode kernel (norm and rotation of q and the new k, the append, the split
 * attention) and, when the attended span is split, a combine kernel.
 *   q          bf16 [B][32][128] new token's queries (before norm and rotation)
 *   k, v       bf16 [B][4][128]  new token's keys and values
 *   q_gain, k_gain  bf16 [128]   RMSNorm gains
 *   sinks      fp32 [32] per query head, or NULL for no sink
 *   pos        int32 [B] device memory: the new token's position, 0 <= pos < cap
 *              and pos + 1 <= max_len (values outside [0, cap) are clamped)
 *   out        bf16 [B][32][128]
 *   workspace  moe_attn_workspace_size(d, B, max_len) bytes, 256 B aligned
 * All pointers are device pointers; q, k, v, the caches and the workspace 16 B
 * aligned, the others aligned to their element.  0 <= B <= 65535; B = 0 is a
 * no-op.  Bad arguments return MOE_ERR_INVALID_ARG (MOE_ERR_WORKSPACE for a
 * short workspace) before anything is enqueued. */
moe_status moe_attn_decode(const moe_attn_desc* d, int32_t B, int32_t max_len, const void* q, const void* k,
                           const void* v, const void* q_gain, const void* k_gain, const float* sinks,
                           const int32_t* pos, void* k_cache, void* v_cache_t, int32_t cap, void* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
