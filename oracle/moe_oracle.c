/*
 * CPU ORACLE for the sparse MoE-layer forward pass -- TEST INFRASTRUCTURE.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg call it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (the method, as the Recursive Flint 40B-A2.5B review by
 * orcarouter.ai states it in "The architecture is an argument about memory
 * bandwidth"): each MoE layer has 256 routed experts of which 6 are chosen per
 * token, plus one shared expert that every token uses; 47 such layers are
 * stacked.  The weight formats (q4_1 and NVFP4 4-bit files, a BF16 checkpoint)
 * are the ones listed in "What actually shipped".  Width, activation, router
 * form and block layouts are not on the page; the readings taken are:
 *   - router: logits = x Wr^T (+ b), fp64 here;
 *   - selection: the k largest logits, ties to the lower expert id;
 *   - weights: softmax over the selected logits (renormalised top-k), or the
 *     top-k entries of the softmax over all experts when renormalisation is off;
 *   - expert: SwiGLU, y = Wd (silu(Wg x) * (Wu x)), silu(g) = g / (1 + e^-g);
 *   - output: sum_j w_j y_{e_j} + shared_scale * y_shared;
 *   - stack: pre-norm residual, r <- r + bf16(MoE(bf16(RMSNorm(r)))), gain 1,
 *     eps inside the square root; output bf16(r).
 * Stored weights are decoded to fp32 exactly as their format defines, then
 * every product and sum is accumulated in fp64 in plain ascending order.
 *
 * Parity pins (all checked by the CPU tests): every decoder against its format
 * definition exhaustively; top-k against brute-force subset search; weights
 * against the softmax identity; the layer against a dense all-experts
 * evaluation and, for one expert, against a numpy SwiGLU; buckets against a
 * key sort; RMSNorm against numpy.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_Q4_1 = 1, ORC_NVFP4 = 2 };

/* One stored matrix set [n][rows][cols]; pointers are host memory. */
typedef struct {
  int32_t fmt;
  int32_t rows, cols;
  const uint8_t* codes;   /* q4_1/NVFP4: [n][rows][cols/2] nibbles; bf16: uint16 [n][rows][cols] */
  const uint16_t* dm;     /* q4_1: fp16 {d, m} per 32-block: [n][rows][cols/32][2] */
  const uint8_t* e4m3;    /* NVFP4: one E4M3 byte per 16-block: [n][rows][cols/16] */
  const float* ts;        /* NVFP4: fp32 per matrix: [n] */
} orc_mat;

typedef struct {
  int32_t d, E, k, f, n_shared, renorm;
  double shared_scale;
  const uint16_t* router_w; /* bf16 [E][d] */
  const float* router_b;    /* fp32 [E] or NULL */
  orc_mat gate, up, down;   /* routed: [E][f][d], [E][f][d], [E][d][f] */
  orc_mat sh_gate, sh_up, sh_down; /* shared: n = 1 */
} orc_layer;

/* ---- number formats, decoded from their definitions ---------------------- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double orc_fp16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double orc_bf16_value(uint16_t b) {
  int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
  double v;
  if (e == 0) v = ldexp((double)m, -133);
  else if (e == 255) v = m ? NAN : INFINITY;
  else v = ldexp(1.0 + (double)m / 128.0, e - 127);
  return s ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; no infinities;
 * S.1111.111 is NaN; exponent 0 is subnormal (m/8) * 2^-6. */
double orc_e4m3_value(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
  double v;
  if (e == 15 && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* FP4 E2M1: bit 3 sign, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent 0 is subnormal m * 0.5. */
double orc_e2m1_value(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* Round a double to the nearest bfloat16 (ties to even); returns the bits. */
uint16_t orc_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0) return sign;
  int ex;
  frexp(a, &ex);               /* a in [2^(ex-1), 2^ex) */
  int q = ex - 8;              /* spacing of 8 significant bits */
  if (q < -133) q = -133;      /* subnormal spacing */
  double r = ldexp(nearbyint(ldexp(a, -q)), q); /* nearbyint: ties to even */
  if (r > 0x1.fep127) return sign | 0x7F80;      /* rounded past the largest finite bf16 */
  /* r is an exact bf16 value: read its bits through fp32 */
  float rf = (float)r;
  uint32_t u;
  memcpy(&u, &rf, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ---- decode tables (built from the formulas above at load time) ---------- */
static double T_FP16[65536], T_BF16[65536], T_E4M3[256], T_E2M1[16];

__attribute__((constructor)) static void orc_tables(void) {
  for (int i = 0; i < 65536; ++i) { T_FP16[i] = orc_fp16_value((uint16_t)i); T_BF16[i] = orc_bf16_value((uint16_t)i); }
  for (int i = 0; i < 256; ++i) T_E4M3[i] = orc_e4m3_value((uint8_t)i);
  for (int i = 0; i < 16; ++i) T_E2M1[i] = orc_e2m1_value((uint8_t)i);
}

/* Position of the scales of 32-element block k within a row of C such blocks:
 * blocks are stored in the order k mod G, then floor(k / G), with G = 16 where
 * 16 divides C and G = C otherwise (the natural order). */
static int64_t orc_scale_pos(int64_t k, int64_t C) {
  const int64_t G = (C % 16 == 0) ? 16 : C;
  return (k % G) * (C / G) + k / G;
}

/* Weight (r, c) of matrix `n` of a stored set, decoded to fp32:
 *   q4_1 : fp32(d) * fp32(q) + fp32(m)  (the product is exact, the add rounds once)
 *   NVFP4: fp32(E2M1 * E4M3) * ts        (the first product is exact)
 *   bf16 : exact widening. */
float orc_weight(const orc_mat* M, int64_t n, int64_t r, int64_t c) {
  int64_t R = M->rows, C = M->cols;
  if (M->fmt == ORC_BF16) {
    const uint16_t* w = (const uint16_t*)M->codes;
    return (float)T_BF16[w[(n * R + r) * C + c]];
  }
  uint8_t byte = M->codes[((n * R + r) * C + c) / 2];
  uint8_t q = (c & 1) ? (byte >> 4) : (byte & 15);
  if (M->fmt == ORC_Q4_1) {
    int64_t blk = (n * R + r) * (C / 32) + orc_scale_pos(c / 32, C / 32);
    float d = (float)T_FP16[M->dm[2 * blk]];
    float m = (float)T_FP16[M->dm[2 * blk + 1]];
    float p = d * (float)q;
    return p + m;
  }
  /* NVFP4 */
  int64_t blk = (n * R + r) * (C / 16) + 2 * orc_scale_pos(c / 32, C / 32) + (c / 16) % 2;
  float p = (float)(T_E2M1[q] * T_E4M3[M->e4m3[blk]]);
  return p * M->ts[n];
}

/* ---- the layer, step by step ------------------------------------------------ */

/* logits[e] = sum_k x[k] * Wr[e][k] (+ b[e]), fp64, k ascending. */
/* All weights of matrix n, decoded (O1), into out[rows][cols]. */
void orc_decode_matrix(const orc_mat* M, int64_t n, float* out) {
  for (int64_t r = 0; r < M->rows; ++r)
    for (int64_t c = 0; c < M->cols; ++c) out[r * M->cols + c] = orc_weight(M, n, r, c);
}

void orc_router_logits(const orc_layer* L, const double* x, double* logits) {
  for (int e = 0; e < L->E; ++e) {
    double s = 0;
    const uint16_t* w = L->router_w + (int64_t)e * L->d;
    for (int k = 0; k < L->d; ++k) s += x[k] * T_BF16[w[k]];
    if (L->router_b) s += (double)L->router_b[e];
    logits[e] = s;
  }
}

typedef struct { double v; int32_t id; } orc_pair;

static int cmp_desc(const void* a, const void* b) {
  const orc_pair* p = (const orc_pair*)a;
  const orc_pair* q = (const orc_pair*)b;
  if (p->v > q->v) return -1;
  if (p->v < q->v) return 1;
  return (p->id > q->id) - (p->id < q->id);
}

/* The k largest logits, ordered (logit descending, id ascending).  gap =
 * (k-th largest) - ((k+1)-th largest), or +inf when k == E. */
void orc_topk(const double* logits, int E, int k, int32_t* ids, double* gap) {
  orc_pair* p = (orc_pair*)malloc(sizeof(orc_pair) * E);
  for (int e = 0; e < E; ++e) { p[e].v = logits[e]; p[e].id = e; }
  qsort(p, E, sizeof(orc_pair), cmp_desc);
  for (int j = 0; j < k; ++j) ids[j] = p[j].id;
  if (gap) *gap = (k < E) ? p[k - 1].v - p[k].v : INFINITY;
  free(p);
}

/* Routing weights of the chosen ids.  renorm: softmax over the chosen
 * logits; otherwise softmax over all E logits, read at the chosen ids. */
void orc_route_weights(const double* logits, int E, const int32_t* ids, int k, int renorm, double* w) {
  double mx = -INFINITY, den = 0;
  if (renorm) {
    for (int j = 0; j < k; ++j) if (logits[ids[j]] > mx) mx = logits[ids[j]];
    for (int j = 0; j < k; ++j) den += exp(logits[ids[j]] - mx);
  } else {
    for (int e = 0; e < E; ++e) if (logits[e] > mx) mx = logits[e];
    for (int e = 0; e < E; ++e) den += exp(logits[e] - mx);
  }
  for (int j = 0; j < k; ++j) w[j] = exp(logits[ids[j]] - mx) / den;
}

/* One SwiGLU expert (matrix index n of the given sets) on one fp64 input row:
 * g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h.  y has L->d entries. */
void orc_expert(const orc_layer* L, const orc_mat* G, const orc_mat* U, const orc_mat* D, int64_t n,
                const double* x, double* y) {
  int d = L->d, f = L->f;
  double* h = (double*)malloc(sizeof(double) * f);
  for (int j = 0; j < f; ++j) {
    double g = 0, u = 0;
    for (int k = 0; k < d; ++k) {
      g += (double)orc_weight(G, n, j, k) * x[k];
      u += (double)orc_weight(U, n, j, k) * x[k];
    }
    h[j] = g / (1.0 + exp(-g)) * u;
  }
  for (int i = 0; i < d; ++i) {
    double s = 0;
    for (int j = 0; j < f; ++j) s += (double)orc_weight(D, n, i, j) * h[j];
    y[i] = s;
  }
  free(h);
}

/* One token through the layer.  x: fp64 [d].  If forced_ids is non-NULL the
 * selection is taken from it instead of from the logits (used to re-evaluate
 * a near-tie token with the other valid choice).  Outputs: out [d], ids [k],
 * w [k], logits [E] (optional), gap (optional). */
void orc_token(const orc_layer* L, const double* x, const int32_t* forced_ids, double* out, int32_t* ids, double* w,
               double* logits_out, double* gap) {
  int E = L->E, k = L->k, d = L->d;
  double* logits = (double*)malloc(sizeof(double) * E);
  double* y = (double*)malloc(sizeof(double) * d);
  orc_router_logits(L, x, logits);
  double g;
  orc_topk(logits, E, k, ids, &g);
  if (forced_ids) memcpy(ids, forced_ids, sizeof(int32_t) * k);
  orc_route_weights(logits, E, ids, k, L->renorm, w);
  for (int i = 0; i < d; ++i) out[i] = 0;
  for (int j = 0; j < k; ++j) {
    orc_expert(L, &L->gate, &L->up, &L->down, ids[j], x, y);
    for (int i = 0; i < d; ++i) out[i] += w[j] * y[i];
  }
  if (L->n_shared) {
    orc_expert(L, &L->sh_gate, &L->sh_up, &L->sh_down, 0, x, y);
    for (int i = 0; i < d; ++i) out[i] += L->shared_scale * y[i];
  }
  if (logits_out) memcpy(logits_out, logits, sizeof(double) * E);
  if (gap) *gap = g;
  free(logits);
  free(y);
}

static int orc_threads(int nthreads) {
#ifdef _OPENMP
  return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* The layer on T bf16 tokens (tokens are independent; threads split them).
 * out: fp64 [T][d]; ids/w: [T][k]; logits [T][E], gaps [T] optional;
 * forced_ids [T][k] optional. */
void orc_layer_forward(const orc_layer* L, const uint16_t* x, int T, const int32_t* forced_ids, double* out,
                       int32_t* ids, double* w, double* logits, double* gaps, int nthreads) {
  int d = L->d, k = L->k, E = L->E;
  int nt = orc_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int t = 0; t < T; ++t) {
    double* xd = (double*)malloc(sizeof(double) * d);
    for (int i = 0; i < d; ++i) xd[i] = T_BF16[x[(int64_t)t * d + i]];
    orc_token(L, xd, forced_ids ? forced_ids + (int64_t)t * k : NULL, out + (int64_t)t * d, ids + (int64_t)t * k,
              w + (int64_t)t * k, logits ? logits + (int64_t)t * E : NULL, gaps ? gaps + t : NULL);
    free(xd);
  }
}

/* Routing only (logits, selection, weights, gaps) for T bf16 tokens. */
void orc_route(const orc_layer* L, const uint16_t* x, int T, int32_t* ids, double* w, double* logits, double* gaps,
               int nthreads) {
  int d = L->d, k = L->k, E = L->E;
  int nt = orc_threads(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
  for (int t = 0; t < T; ++t) {
    double* xd = (double*)malloc(sizeof(double) * d);
    double* lg = (double*)malloc(sizeof(double) * E);
    for (int i = 0; i < d; ++i) xd[i] = T_BF16[x[(int64_t)t * d + i]];
    orc_router_logits(L, xd, lg);
    double g;
    orc_topk(lg, E, k, ids + (int64_t)t * k, &g);
    orc_route_weights(lg, E, ids + (int64_t)t * k, k, L->renorm, w + (int64_t)t * k);
    if (logits) memcpy(logits + (int64_t)t * E, lg, sizeof(double) * E);
    if (gaps) gaps[t] = g;
    free(xd);
    free(lg);
  }
}

/* ---- expert buckets ---------------------------------------------------------- */

typedef struct { int32_t key, slot; } orc_ks;
static int cmp_ks(const void* a, const void* b) {
  const orc_ks* p = (const orc_ks*)a;
  const orc_ks* q = (const orc_ks*)b;
  if (p->key != q->key) return (p->key > q->key) - (p->key < q->key);
  return (p->slot > q->slot) - (p->slot < q->slot);
}

/* Slots s = t*k + j carry expert ids[s].  counts[e] = #slots with id e;
 * offsets = exclusive prefix sum (offsets[E] = T*k); perm = slot indices
 * sorted by (id, slot), i.e. a stable sort by id; inv_perm its inverse. */
void orc_buckets(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv_perm) {
  int S = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int s = 0; s < S; ++s) counts[ids[s]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  orc_ks* v = (orc_ks*)malloc(sizeof(orc_ks) * (S > 0 ? S : 1));
  for (int s = 0; s < S; ++s) { v[s].key = ids[s]; v[s].slot = s; }
  qsort(v, S, sizeof(orc_ks), cmp_ks);
  for (int p = 0; p < S; ++p) { perm[p] = v[p].slot; inv_perm[v[p].slot] = p; }
  free(v);
}

/* ---- the stack --------------------------------------------------------------- */

/* RMSNorm of one fp64 row with gain 1: r / sqrt(mean(r^2) + eps), each entry
 * rounded to bf16 (the layer input is a bf16 tensor). */
void orc_rmsnorm_bf16(const double* r, int d, double eps, uint16_t* out) {
  double ss = 0;
  for (int i = 0; i < d; ++i) ss += r[i] * r[i];
  double inv = 1.0 / sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) out[i] = orc_bf16_rne(r[i] * inv);
}

/* n_layers MoE layers on T tokens: r0 = x; for each layer l,
 * xn = bf16(RMSNorm(r)); y = layer_l(xn); r = r + bf16(y).  Output bf16(r).
 * Records (optional): xin [n_layers][T][d] bf16 layer inputs, yout
 * [n_layers][T][d] bf16 layer outputs, ids [n_layers][T][k]. */
void orc_stack_forward(const orc_layer* const* layers, int n_layers, const uint16_t* x, int T, double eps,
                       uint16_t* out, uint16_t* xin_rec, uint16_t* yout_rec, int32_t* ids_rec, int nthreads) {
  if (n_layers <= 0 || T <= 0) return;
  int d = layers[0]->d;
  int nt = orc_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int t = 0; t < T; ++t) {
    double* r = (double*)malloc(sizeof(double) * d);
    double* xd = (double*)malloc(sizeof(double) * d);
    double* y = (double*)malloc(sizeof(double) * d);
    uint16_t* xn = (uint16_t*)malloc(sizeof(uint16_t) * d);
    int32_t ids[64];
    double w[64];
    for (int i = 0; i < d; ++i) r[i] = T_BF16[x[(int64_t)t * d + i]];
    for (int l = 0; l < n_layers; ++l) {
      const orc_layer* L = layers[l];
      orc_rmsnorm_bf16(r, d, eps, xn);
      for (int i = 0; i < d; ++i) xd[i] = T_BF16[xn[i]];
      orc_token(L, xd, NULL, y, ids, w, NULL, NULL);
      for (int i = 0; i < d; ++i) {
        uint16_t yb = orc_bf16_rne(y[i]);
        r[i] += T_BF16[yb];
        if (yout_rec) yout_rec[((int64_t)l * T + t) * d + i] = yb;
      }
      if (xin_rec) memcpy(xin_rec + ((int64_t)l * T + t) * d, xn, sizeof(uint16_t) * d);
      if (ids_rec) memcpy(ids_rec + ((int64_t)l * T + t) * L->k, ids, sizeof(int32_t) * L->k);
    }
    for (int i = 0; i < d; ++i) out[(int64_t)t * d + i] = orc_bf16_rne(r[i]);
    free(r); free(xd); free(y); free(xn);
  }
}

/* Output head (the 4-bit lm_head of "The quantisation recipe is the most
 * transferable part"): logits[t][v] = sum_k x[t][k] w[v][k] for the stored
 * matrix W (n = 0, rows = vocabulary, cols = d) and bf16 tokens x [T][cols].
 * rows: the vocabulary rows to evaluate (n_rows of them; NULL = all rows in
 * order); out: fp64 [T][n_rows].  Each row is decoded once, then dotted with
 * every token in ascending k. */
void orc_head_logits(const orc_mat* W, const uint16_t* x, int T, const int32_t* rows, int n_rows, double* out,
                     int nthreads) {
  int d = W->cols;
  double* xd = (double*)malloc(sizeof(double) * ((int64_t)T * d + 1));
  for (int64_t i = 0; i < (int64_t)T * d; ++i) xd[i] = T_BF16[x[i]];
  int nt = orc_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
  for (int i = 0; i < n_rows; ++i) {
    int64_t v = rows ? rows[i] : i;
    double* wr = (double*)malloc(sizeof(double) * d);
    for (int k = 0; k < d; ++k) wr[k] = (double)orc_weight(W, 0, v, k);
    for (int t = 0; t < T; ++t) {
      const double* xt = xd + (int64_t)t * d;
      double s = 0.0;
      for (int k = 0; k < d; ++k) s += wr[k] * xt[k];
      out[(int64_t)t * n_rows + i] = s;
    }
    free(wr);
  }
  free(xd);
}

/* ---- decode attention ----------------------------------------------------------
 * The attention layout of "The architecture is an argument about memory
 * bandwidth": 32 query heads and 4 key-value heads of dimension 128 (query
 * head h reads key-value head h / 8); sliding-window layers attend to the
 * current token and the 512 before it (a window of 513), the other layers to
 * every earlier token; rotary position embedding on the sliding-window layers
 * only; an RMSNorm over each head of q and k; a learned sink per query head.
 * Readings (the pages give no formulas): RMSNorm x / sqrt(mean(x^2) + eps) *
 * gain; the norm comes before the rotation; the rotation pairs element i with
 * i + D/2 at angle pos * theta^(-2i/D); scores q.k / sqrt(D); the sink z_h is
 * one more logit in the softmax's denominator with no value. */

/* Per-head RMSNorm then (if rope) rotation of one head vector x[D] at position
 * pos; result in y (fp64). */
static void orc_qk_head(const double* x, int D, const double* gain, double eps, int rope, double theta, int64_t pos,
                        double* y) {
  double ss = 0.0;
  for (int i = 0; i < D; ++i) ss += x[i] * x[i];
  const double r = 1.0 / sqrt(ss / D + eps);
  for (int i = 0; i < D; ++i) y[i] = x[i] * r * gain[i];
  if (!rope) return;
  const int H = D / 2;
  for (int i = 0; i < H; ++i) {
    const double ang = (double)pos * pow(theta, -2.0 * i / D);
    const double c = cos(ang), s = sin(ang), a = y[i], b = y[i + H];
    y[i] = a * c - b * s;
    y[i + H] = b * c + a * s;
  }
}

/* The new token's q and k: normalised, rotated (if rope) and rounded to bf16.
 * q [B][HQ][D], k [B][HK][D] bf16 in; gains [D] (bf16); pos [B]; outputs bf16. */
void orc_attn_prep(const uint16_t* q, const uint16_t* k, int B, int HQ, int HK, int D, const uint16_t* q_gain,
                   const uint16_t* k_gain, const int32_t* pos, int rope, double theta, double eps, uint16_t* q_out,
                   uint16_t* k_out) {
  double* x = (double*)malloc(sizeof(double) * D);
  double* y = (double*)malloc(sizeof(double) * D);
  double* gq = (double*)malloc(sizeof(double) * D);
  double* gk = (double*)malloc(sizeof(double) * D);
  for (int i = 0; i < D; ++i) { gq[i] = T_BF16[q_gain[i]]; gk[i] = T_BF16[k_gain[i]]; }
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < HQ + HK; ++h) {
      const int isq = h < HQ;
      const uint16_t* src = isq ? q + ((int64_t)b * HQ + h) * D : k + ((int64_t)b * HK + (h - HQ)) * D;
      uint16_t* dst = isq ? q_out + ((int64_t)b * HQ + h) * D : k_out + ((int64_t)b * HK + (h - HQ)) * D;
      for (int i = 0; i < D; ++i) x[i] = T_BF16[src[i]];
      orc_qk_head(x, D, isq ? gq : gk, eps, rope, theta, pos[b], y);
      for (int i = 0; i < D; ++i) dst[i] = orc_bf16_rne(y[i]);
    }
  }
  free(x); free(y); free(gq); free(gk);
}

/* Attention of one new token per sequence over its cache.
 * q [B][HQ][D] bf16 (prepared); kc, vc [B][cap][HK][D] bf16, positions 0 ..
 * len[b]-1 valid; window 0 = every position, else the last `window` ones;
 * sinks [HQ] fp32 or NULL (no sink); out [B][HQ][D] fp64.  Each (b, h) is an
 * independent softmax; threads split them. */
void orc_attn_decode(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* len, int B, int HQ,
                     int HK, int D, int cap, int window, const float* sinks, double* out, int nthreads) {
  int nt = orc_threads(nthreads);
  const int G = HQ / HK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int bh = 0; bh < B * HQ; ++bh) {
    const int b = bh / HQ, h = bh % HQ, kv = h / G;
    const int n = len[b];
    const int lo = (window > 0 && n > window) ? n - window : 0;
    double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
    const uint16_t* qh = q + ((int64_t)b * HQ + h) * D;
    double m = -INFINITY;
    for (int p = lo; p < n; ++p) {
      const uint16_t* kp = kc + (((int64_t)b * cap + p) * HK + kv) * D;
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += T_BF16[qh[i]] * T_BF16[kp[i]];
      s[p - lo] = acc / sqrt((double)D);
      if (s[p - lo] > m) m = s[p - lo];
    }
    const double z = sinks ? (double)sinks[h] : -INFINITY;
    if (z > m) m = z;
    double den = sinks ? exp(z - m) : 0.0;
    for (int p = lo; p < n; ++p) den += exp(s[p - lo] - m);
    double* o = out + ((int64_t)b * HQ + h) * D;
    for (int i = 0; i < D; ++i) o[i] = 0.0;
    for (int p = lo; p < n; ++p) {
      const double w = exp(s[p - lo] - m) / den;
      const uint16_t* vp = vc + (((int64_t)b * cap + p) * HK + kv) * D;
      for (int i = 0; i < D; ++i) o[i] += w * T_BF16[vp[i]];
    }
    free(s);
  }
}

int orc_max_threads(void) { return orc_threads(0); }
