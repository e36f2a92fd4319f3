/*
 * synth.c -- fast, seeded synthesis of workload inputs (multi-threaded).
 *
 * Input generation only: normal samples from a counter-based generator and
 * their encodings into the storage formats the GEMMs consume.  No GEMM,
 * accumulation or decode-for-compute arithmetic lives here.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014; constants as published by Vigna)
 * applied to (key + counter), two 53-bit uniforms per Box-Muller pair.  The
 * value at index i depends only on (key, i), so any thread split gives the
 * same tensor.
 *
 * Encodings (the formats' usual definitions):
 *   E4M3-FN  round to nearest even, saturate at +-448
 *   E2M1     round to nearest even on {0,.5,1,1.5,2,3,4,6}, saturate at 6
 *   NVFP4    S = amax/(448*6) (1 if zero); group-of-16 scale RNE_E4M3(amax_g/6/S);
 *            codes RNE_E2M1(x/(scale*S)); element 2i in the low nibble
 *   FP8 tok  s = amax_row/448 (1 if zero); codes RNE_E4M3(x/s)
 *   MXFP8    per 32: X = floor(log2 amax) - 8 in [-127,127], byte X+127
 *            (0 for an all-zero block), codes RNE_E4M3(x/2^X)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t sm64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

uint64_t syn_key(uint64_t seed, uint64_t role) {
  return sm64(sm64(seed) ^ sm64(0xD1B54A32D192ED03ull * (role + 1)));
}

/* -------------------------------------------------------------- threads */
typedef struct {
  void (*fn)(void *, int64_t, int64_t);
  void *ctx;
  int64_t lo, hi;
} job_t;

static void *run_job(void *p) {
  job_t *j = (job_t *)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void par(int64_t n, int nth, void *ctx, void (*fn)(void *, int64_t, int64_t)) {
  if (nth < 1) nth = 1;
  if (nth > 64) nth = 64;
  if (n < nth) nth = n > 0 ? (int)n : 1;
  pthread_t th[64];
  job_t jb[64];
  int ok[64];
  for (int i = 0; i < nth; i++) {
    jb[i].fn = fn;
    jb[i].ctx = ctx;
    jb[i].lo = n * i / nth;
    jb[i].hi = n * (i + 1) / nth;
    ok[i] = nth > 1 && pthread_create(&th[i], NULL, run_job, &jb[i]) == 0;
    if (!ok[i]) run_job(&jb[i]);
  }
  for (int i = 0; i < nth; i++)
    if (ok[i]) pthread_join(th[i], NULL);
}

/* --------------------------------------------------------------- normal */
typedef struct {
  uint64_t key;
  float std;
  float *out;
  int64_t n;
} normal_ctx;

static void normal_range(void *p, int64_t lo, int64_t hi) {
  normal_ctx *c = (normal_ctx *)p;
  /* pairs j cover indices 2j, 2j+1 */
  for (int64_t j = lo; j < hi; j++) {
    uint64_t r1 = sm64(c->key + 2 * (uint64_t)j), r2 = sm64(c->key + 2 * (uint64_t)j + 1);
    double u1 = ((double)(r1 >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0,1] */
    double u2 = (double)(r2 >> 11) * (1.0 / 9007199254740992.0);         /* [0,1) */
    double rad = sqrt(-2.0 * log(u1)), ang = 6.283185307179586 * u2;
    int64_t i = 2 * j;
    c->out[i] = (float)(rad * cos(ang)) * c->std;
    if (i + 1 < c->n) c->out[i + 1] = (float)(rad * sin(ang)) * c->std;
  }
}

void syn_normal(uint64_t key, float std, float *out, int64_t n, int nth) {
  normal_ctx c = {key, std, out, n};
  par((n + 1) / 2, nth, &c, normal_range);
}

/* ------------------------------------------------------------- encoders */
static uint8_t enc_e4m3(double v) {
  if (v != v) return 0x7F;
  uint8_t s = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return s | 0x7E;
  if (a == 0.0) return s;
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  if (e < -6) e = -6;
  double step = ldexp(1.0, e - 3);
  double r = nearbyint(a / step) * step;
  if (r >= 448.0) return s | 0x7E;
  if (r == 0.0) return s;
  if (r < 0.015625) return s | (uint8_t)nearbyint(r * 512.0);
  frexp(r, &ex);
  int er = ex - 1;
  int m = (int)nearbyint((ldexp(r, -er) - 1.0) * 8.0);
  return s | (uint8_t)(((er + 7) << 3) | m);
}

static double dec_e4m3(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp((double)m, -9);
  return (b & 0x80) ? -v : v;
}

static uint8_t enc_e2m1(double x) {
  double a = fabs(x);
  int idx;
  /* nearest on {0,.5,1,1.5,2,3,4,6}; ties to the even code (mantissa bit 0) */
  if (a <= 0.25) idx = 0;
  else if (a < 0.75) idx = 1;
  else if (a <= 1.25) idx = 2;
  else if (a < 1.75) idx = 3;
  else if (a <= 2.5) idx = 4;
  else if (a < 3.5) idx = 5;
  else if (a <= 5.0) idx = 6;
  else idx = 7;
  return (uint8_t)(idx | ((signbit(x) && idx) ? 8 : 0));
}

/* --------------------------------------------------------------- amax */
typedef struct {
  const float *x;
  int64_t n;
  float part[64];
  int64_t chunk;
} amax_ctx;

static void amax_range(void *p, int64_t lo, int64_t hi) {
  amax_ctx *c = (amax_ctx *)p;
  for (int64_t t = lo; t < hi; t++) {
    float m = 0.0f;
    int64_t a = t * c->chunk, b = a + c->chunk < c->n ? a + c->chunk : c->n;
    for (int64_t i = a; i < b; i++) {
      float v = fabsf(c->x[i]);
      if (v > m) m = v;
    }
    c->part[t] = m;
  }
}

float syn_amax(const float *x, int64_t n, int nth) {
  amax_ctx c;
  c.x = x;
  c.n = n;
  c.chunk = (n + 63) / 64;
  if (c.chunk < 1) c.chunk = 1;
  int64_t nt = (n + c.chunk - 1) / c.chunk;
  par(nt, nth, &c, amax_range);
  float m = 0.0f;
  for (int64_t t = 0; t < nt; t++)
    if (c.part[t] > m) m = c.part[t];
  return m;
}

/* ---------------------------------------------------------------- NVFP4 */
typedef struct {
  const float *x;
  int64_t K;
  double S;
  uint8_t *codes, *scales;
} nv_ctx;

static void nv_range(void *p, int64_t lo, int64_t hi) {
  nv_ctx *c = (nv_ctx *)p;
  const int64_t G = c->K / 16;
  for (int64_t r = lo; r < hi; r++)
    for (int64_t g = 0; g < G; g++) {
      const float *v = c->x + r * c->K + 16 * g;
      double am = 0.0;
      for (int i = 0; i < 16; i++)
        if (fabs((double)v[i]) > am) am = fabs((double)v[i]);
      uint8_t sb = enc_e4m3(am / 6.0 / c->S);
      double div = dec_e4m3(sb) * c->S;
      c->scales[r * G + g] = sb;
      uint8_t *q = c->codes + r * (c->K / 2) + 8 * g;
      for (int i = 0; i < 8; i++) {
        uint8_t lo4 = div == 0.0 ? 0 : enc_e2m1((double)v[2 * i] / div);
        uint8_t hi4 = div == 0.0 ? 0 : enc_e2m1((double)v[2 * i + 1] / div);
        q[i] = (uint8_t)(lo4 | (hi4 << 4));
      }
    }
}

/* returns the tensor scale S */
float syn_quant_nvfp4(const float *x, int64_t R, int64_t K, uint8_t *codes, uint8_t *scales,
                      int nth) {
  float amax = syn_amax(x, R * K, nth);
  float S = amax > 0.0f ? (float)((double)amax / (448.0 * 6.0)) : 1.0f;
  if (S == 0.0f) S = 1.0f;
  nv_ctx c = {x, K, (double)S, codes, scales};
  par(R, nth, &c, nv_range);
  return S;
}

/* ------------------------------------------------------------ FP8 token */
typedef struct {
  const float *x;
  int64_t K;
  uint8_t *q;
  float *s;
} tok_ctx;

static void tok_range(void *p, int64_t lo, int64_t hi) {
  tok_ctx *c = (tok_ctx *)p;
  for (int64_t r = lo; r < hi; r++) {
    const float *v = c->x + r * c->K;
    float am = 0.0f;
    for (int64_t k = 0; k < c->K; k++)
      if (fabsf(v[k]) > am) am = fabsf(v[k]);
    float s = am > 0.0f ? am / 448.0f : 1.0f;
    c->s[r] = s;
    for (int64_t k = 0; k < c->K; k++) c->q[r * c->K + k] = enc_e4m3((double)v[k] / (double)s);
  }
}

void syn_quant_fp8_token(const float *x, int64_t M, int64_t K, uint8_t *q, float *s, int nth) {
  tok_ctx c = {x, K, q, s};
  par(M, nth, &c, tok_range);
}

/* ---------------------------------------------------------------- MXFP8 */
typedef struct {
  const float *x;
  uint8_t *codes, *scales;
} mx_ctx;

static void mx_range(void *p, int64_t lo, int64_t hi) {
  mx_ctx *c = (mx_ctx *)p;
  for (int64_t b = lo; b < hi; b++) {
    const float *v = c->x + 32 * b;
    double am = 0.0;
    for (int i = 0; i < 32; i++)
      if (fabs((double)v[i]) > am) am = fabs((double)v[i]);
    int X = -127;
    if (am > 0.0) {
      int ex;
      frexp(am, &ex);
      X = ex - 1 - 8;
      if (X < -127) X = -127;
      if (X > 127) X = 127;
    }
    c->scales[b] = (uint8_t)(X + 127);
    for (int i = 0; i < 32; i++) c->codes[32 * b + i] = enc_e4m3(ldexp((double)v[i], -X));
  }
}

void syn_quant_mxfp8(const float *x, int64_t n, uint8_t *codes, uint8_t *scales, int nth) {
  mx_ctx c = {x, codes, scales};
  par(n / 32, nth, &c, mx_range);
}

/* ----------------------------------------------------------------- BF16 */
typedef struct {
  const float *x;
  uint16_t *out;
} bf_ctx;

static void bf_range(void *p, int64_t lo, int64_t hi) {
  bf_ctx *c = (bf_ctx *)p;
  for (int64_t i = lo; i < hi; i++) {
    uint32_t u;
    memcpy(&u, &c->x[i], 4);
    c->out[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  }
}

void syn_to_bf16(const float *x, int64_t n, uint16_t *out, int nth) {
  bf_ctx c = {x, out};
  par(n, nth, &c, bf_range);
}
