/*
 * Seeded synthetic inputs for the MoE-layer path: random draws, and the
 * encoders that store drawn weights in the library's 4-bit layouts.
 *
 * This module only PRODUCES inputs (activations, router weights, router bias,
 * packed expert weights).  It contains none of the forward arithmetic: no
 * decoding of stored weights back to numbers for a matmul, no routing, no FFN.
 * The CPU oracle and the HIP library both consume the bytes it writes, and
 * neither of them links this file.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output of the
 * generator seeded with s is mix(s + (i + 1) * GAMMA), so any element of any
 * stream can be computed independently (counter-based use).  Normals come from
 * the Box-Muller transform on pairs of uniforms.
 *
 * Formats written here (element 2i of a row is the low nibble of byte i):
 *   q4_1  : blocks of 32 along a row; fp16 scale d and fp16 min m per block,
 *           stored interleaved {d, m}; unsigned 4-bit codes q, w = d*q + m.
 *   NVFP4 : blocks of 16 along a row; E2M1 codes (bit 3 = sign), one FP8 E4M3
 *           (OCP E4M3FN) scale per block, one fp32 scale per matrix.
 *   bf16  : plain bf16.
 * The scales of a row are stored in the order of scale_pos() below (per
 * 32-element block; NVFP4 keeps a block's two scales together).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output (0-based) of SplitMix64 seeded with `seed`. */
uint64_t synth_u64(uint64_t seed, uint64_t i) { return sm64_mix(seed + (i + 1) * GAMMA); }

/* Stream key for a (seed, tag, a, b) tuple: chained mixing, so that distinct
 * tuples give unrelated streams. */
uint64_t synth_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b) {
  uint64_t k = sm64_mix(seed * GAMMA + 0x5851F42D4C957F2DULL);
  k = sm64_mix(k ^ (tag * 0xD6E8FEB86659FD93ULL));
  k = sm64_mix(k ^ (a * 0xA0761D6478BD642FULL + 1));
  k = sm64_mix(k ^ (b * 0xE7037ED1A0B428DBULL + 2));
  return k;
}

/* Uniform in the open interval (0, 1): 53 random bits, offset by half a step. */
static inline double u01(uint64_t seed, uint64_t i) {
  return ((double)(synth_u64(seed, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* i-th standard normal of stream `seed` (Box-Muller on uniform pair i/2). */
static inline double normal_at(uint64_t seed, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = u01(seed, 2 * p), u2 = u01(seed, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

/* out[j] = fp32(sigma * N_{start + j}) for j in [0, n), start even, n even:
 * both values of each Box-Muller pair are used. */
static void normals_f32(uint64_t seed, uint64_t start, int64_t n, double sigma, float* out) {
  for (int64_t j = 0; j < n; j += 2) {
    uint64_t p = (start + (uint64_t)j) >> 1;
    double u1 = u01(seed, 2 * p), u2 = u01(seed, 2 * p + 1);
    double r = sqrt(-2.0 * log(u1));
    double sn, cs;
    sincos(6.283185307179586476925286766559 * u2, &sn, &cs);
    out[j] = (float)(sigma * (r * cs));
    out[j + 1] = (float)(sigma * (r * sn));
  }
}

/* ---- rounding helpers (encoders) ---------------------------------------- */

/* fp32 bits -> bf16 bits, round to nearest even (finite inputs). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* double -> fp16 bits, round to nearest even, overflow to inf. */
uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < 0.00006103515625) { /* below 2^-14: subnormal step 2^-24 */
    double q = nearbyint(a * 16777216.0);
    return sign | (uint16_t)q;   /* q == 1024 encodes the smallest normal */
  }
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;           /* a = 1.mant * 2^e */
  double mant = nearbyint((ldexp(f, 1) - 1.0) * 1024.0);
  if (mant >= 1024.0) { mant = 0.0; e += 1; }
  if (e > 15) return sign | 0x7C00;
  return sign | (uint16_t)(((e + 15) << 10) | (int)mant);
}

/* fp16 bits -> double (generator-side decode, used only while encoding). */
static double f16_bits_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v = (e == 0) ? ldexp((double)m, -24) : ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* E4M3 (OCP E4M3FN) value of a byte, generator side. */
static double e4m3_bits_value(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* non-negative double -> E4M3 byte, round to nearest even, saturate at 448. */
uint8_t synth_f64_to_e4m3_sat(double a) {
  if (!(a > 0)) return 0;
  if (a >= 448.0) return 0x7E;
  if (a < 0.015625) { /* below 2^-6: subnormal step 2^-9 */
    double q = nearbyint(a * 512.0);
    return (uint8_t)q; /* q == 8 encodes the smallest normal */
  }
  int ex;
  double f = frexp(a, &ex);
  int e = ex - 1;
  double mant = nearbyint((ldexp(f, 1) - 1.0) * 8.0);
  if (mant >= 8.0) { mant = 0.0; e += 1; }
  int bits = ((e + 7) << 3) | (int)mant;
  if (bits > 0x7E) bits = 0x7E;
  return (uint8_t)bits;
}

/* nearest E2M1 code to v (ties to the even code, magnitude clamped at 6). */
uint8_t synth_f64_to_e2m1(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint8_t sign = (v < 0) ? 8 : 0;
  double a = fabs(v);
  int best = 0;
  double bd = a;
  for (int c = 1; c < 8; ++c) {
    double dd = fabs(a - mag[c]);
    if (dd < bd || (dd == bd && (c & 1) == 0)) { bd = dd; best = c; }
  }
  return sign | (uint8_t)best;
}

/* ---- draws ----------------------------------------------------------------- */

/* out[i] = fp32(sigma * N_i) for i in [0, n). */
void synth_normal_f32(uint64_t key, double sigma, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(sigma * normal_at(key, (uint64_t)i));
}

/* out[i] = bf16(fp32(sigma * N_i)), each rounding to nearest even. */
void synth_normal_bf16(uint64_t key, double sigma, uint16_t* out, int64_t n) {
  int64_t np2 = n & ~(int64_t)1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < np2; i += 2) {
    float v[2];
    normals_f32(key, (uint64_t)i, 2, sigma, v);
    out[i] = f32_to_bf16_rne(v[0]);
    out[i + 1] = f32_to_bf16_rne(v[1]);
  }
  if (n & 1) out[n - 1] = f32_to_bf16_rne((float)(sigma * normal_at(key, (uint64_t)(n - 1))));
}

/* out[i] = the low byte of output i of stream `key`: uniform bytes, for
 * patterned weights that set every code and scale byte directly. */
void synth_bytes(uint64_t key, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)synth_u64(key, (uint64_t)i);
}

/* Random permutation of 0..n-1 (Fisher-Yates with stream `key`). */
void synth_permutation(uint64_t key, int32_t* perm, int32_t n) {
  for (int32_t i = 0; i < n; ++i) perm[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    /* multiply-shift reduction of a 64-bit draw to [0, i] */
    unsigned __int128 p = (unsigned __int128)synth_u64(key, (uint64_t)(n - 1 - i)) * (uint64_t)(i + 1);
    int32_t j = (int32_t)(p >> 64);
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
}

/* ---- encoders -------------------------------------------------------------- */

/* q4_1 encode of one row of `cols` fp32 values (cols % 32 == 0). */
/* Storage order of the scales within a row of C blocks of 32 elements: block k
 * at position (k mod G) * (C / G) + floor(k / G), G = 16 when 16 divides C
 * (else G = C, the identity).  With C = 64 the 16 blocks a lane of the
 * library's vector path reads in one pass of K = 512 lie 4 positions apart, and
 * its 4 blocks k, k + 16, k + 32, k + 48 are adjacent; with C = 16 the order is
 * the natural one. */
static inline int64_t scale_pos(int64_t k, int64_t C) {
  const int64_t G = (C % 16 == 0) ? 16 : C;
  return (k % G) * (C / G) + k / G;
}

static void q4_1_row(const float* w, int64_t cols, uint8_t* codes, uint16_t* dm) {
  for (int64_t b = 0; b < cols / 32; ++b) {
    const float* x = w + 32 * b;
    double mn = x[0], mx = x[0];
    for (int i = 1; i < 32; ++i) { if (x[i] < mn) mn = x[i]; if (x[i] > mx) mx = x[i]; }
    uint16_t mh = synth_f64_to_f16(mn);
    uint16_t dh = synth_f64_to_f16((mx - mn) / 15.0);
    double md = f16_bits_value(mh), dd = f16_bits_value(dh);
    uint8_t q[32];
    for (int i = 0; i < 32; ++i) {
      double t = (dd == 0.0) ? 0.0 : nearbyint(((double)x[i] - md) / dd);
      if (t < 0) t = 0;
      if (t > 15) t = 15;
      q[i] = (uint8_t)t;
    }
    for (int i = 0; i < 16; ++i) codes[16 * b + i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
    const int64_t p = scale_pos(b, cols / 32);
    dm[2 * p] = dh;
    dm[2 * p + 1] = mh;
  }
}

/* q4_1 encode of a rows x cols fp32 matrix. codes: rows*cols/2 bytes,
 * dm: rows*(cols/32)*2 fp16 values ({d, m} per block). */
void synth_q4_1_encode(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* dm) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) q4_1_row(w + r * cols, cols, codes + r * cols / 2, dm + r * (cols / 32) * 2);
}

/* NVFP4 encode of a rows x cols fp32 matrix (cols % 32 == 0; the two scales
 * of a 32-element block are stored together at that block's position).
 * ts = amax/(6*448) in fp32; block scale s = E4M3(amax_b / (6*ts)); code =
 * nearest E2M1 to w / (s*ts).  codes: rows*cols/2 bytes, scales: rows*cols/16. */
void synth_nvfp4_encode(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                        float* tensor_scale) {
  double amax = 0;
  for (int64_t i = 0; i < rows * cols; ++i) { double a = fabs((double)w[i]); if (a > amax) amax = a; }
  float ts = (amax > 0) ? (float)(amax / (6.0 * 448.0)) : 1.0f;
  *tensor_scale = ts;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      const float* x = w + r * cols + 16 * b;
      double ab = 0;
      for (int i = 0; i < 16; ++i) { double a = fabs((double)x[i]); if (a > ab) ab = a; }
      uint8_t s = synth_f64_to_e4m3_sat(ab / (6.0 * (double)ts));
      scales[r * (cols / 16) + 2 * scale_pos(b / 2, cols / 32) + (b & 1)] = s;
      double sv = e4m3_bits_value(s) * (double)ts;
      uint8_t c[16];
      for (int i = 0; i < 16; ++i) c[i] = (sv == 0.0) ? 0 : synth_f64_to_e2m1((double)x[i] / sv);
      for (int i = 0; i < 8; ++i) codes[r * cols / 2 + 8 * b + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    }
  }
}

/* fp32 -> bf16 (RNE) for a whole array. */
void synth_f32_to_bf16(const float* w, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(w[i]);
}

/* Draw-and-encode of one rows x cols matrix, without keeping the fp32 copy
 * beyond one row per thread.  fmt: 0 = bf16, 1 = q4_1, 2 = NVFP4.
 * NVFP4 needs the matrix amax first, so it draws the matrix twice (the draw is
 * counter based, so both passes see the same values). */
void synth_matrix(uint64_t key, double sigma, int fmt, int64_t rows, int64_t cols, void* codes, void* scales,
                  float* tensor_scale) {
  if (fmt == 0) {
    synth_normal_bf16(key, sigma, (uint16_t*)codes, rows * cols);
    return;
  }
  if (fmt == 1) {
#pragma omp parallel
    {
      float* row = (float*)malloc(sizeof(float) * cols);
#pragma omp for schedule(static)
      for (int64_t r = 0; r < rows; ++r) {
        normals_f32(key, (uint64_t)(r * cols), cols, sigma, row);
        q4_1_row(row, cols, (uint8_t*)codes + r * cols / 2, (uint16_t*)scales + r * (cols / 32) * 2);
      }
      free(row);
    }
    return;
  }
  /* NVFP4 */
  double amax = 0;
#pragma omp parallel for schedule(static) reduction(max : amax)
  for (int64_t r = 0; r < rows; ++r) {
    float x[16];
    for (int64_t c = 0; c < cols; c += 16) {
      normals_f32(key, (uint64_t)(r * cols + c), 16, sigma, x);
      for (int i = 0; i < 16; ++i) { double a = fabs((double)x[i]); if (a > amax) amax = a; }
    }
  }
  float ts = (amax > 0) ? (float)(amax / (6.0 * 448.0)) : 1.0f;
  *tensor_scale = ts;
  uint8_t* cd = (uint8_t*)codes;
  uint8_t* sc = (uint8_t*)scales;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      float x[16];
      double ab = 0;
      normals_f32(key, (uint64_t)(r * cols + 16 * b), 16, sigma, x);
      for (int i = 0; i < 16; ++i) {
        double a = fabs((double)x[i]);
        if (a > ab) ab = a;
      }
      uint8_t s = synth_f64_to_e4m3_sat(ab / (6.0 * (double)ts));
      sc[r * (cols / 16) + 2 * scale_pos(b / 2, cols / 32) + (b & 1)] = s;
      double sv = e4m3_bits_value(s) * (double)ts;
      uint8_t c[16];
      for (int i = 0; i < 16; ++i) c[i] = (sv == 0.0) ? 0 : synth_f64_to_e2m1((double)x[i] / sv);
      for (int i = 0; i < 8; ++i) cd[r * cols / 2 + 8 * b + i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    }
  }
}
