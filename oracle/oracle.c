/*
 * oracle.c -- plain FP64 CPU oracle for the block-scaled TN GEMM hot path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product.  Shares no code
 * with the GPU path.  Every value is the plain definition written out: decode
 * each operand element to FP64, multiply, sum in ascending k.  Threads only
 * split independent output points; no blocking or reordering of any sum.
 *
 * Sources (web pages, cited by title and section):
 *  - metrale_circuit "hardware::exec" module documentation, module description:
 *    the declared formats of a weight-reading node, the E2M1 -> E4M3 bit
 *    identity (value times 2^-6 for all 16 codes, the 2^6 folded into the group
 *    scale) and the per-K=16 FP32 block-scale application on the FP8 MMA.
 *  - FlashInfer "swapab_cutedsl_megakernel" skill page, Layout section: the
 *    MXFP8 GLU mixture-of-experts (gate/up, GLU, down) whose generic reference
 *    the MoE functions below restate, and the NVFP4 MoE the page lists beside
 *    it (moe_nvfp4_swapab), whose computation is read here as the same GLU
 *    MoE with every operand in NVFP4 (the orc_moe4_* functions).
 * Format definitions (E2M1, E4M3-FN, E8M0, BF16) are the OCP / IEEE ones; the
 * pages name the formats without defining their bits.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ decode */

double orc_dec_bf16(uint16_t u) {
  /* BF16 is the top half of an IEEE binary32 */
  uint32_t bits = (uint32_t)u << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

double orc_dec_e2m1(uint8_t code) {
  /* sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0 */
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

double orc_dec_e4m3(uint8_t b) {
  /* OCP E4M3-FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0;
     exponent 15 with mantissa 7 is NaN; no infinities */
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

double orc_dec_e8m0(uint8_t x) {
  if (x == 255) return NAN;
  return ldexp(1.0, (int)x - 127);
}

double orc_elem(const orc_operand *x, int64_t r, int64_t k) {
  const int64_t K = x->K;
  switch (x->fmt) {
    case ORC_BF16:
      return orc_dec_bf16(((const uint16_t *)x->data)[r * K + k]);
    case ORC_NVFP4: {
      uint8_t byte = ((const uint8_t *)x->data)[r * (K / 2) + k / 2];
      uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
      return orc_dec_e2m1(code) * orc_dec_e4m3(x->scales[r * (K / 16) + k / 16]);
    }
    case ORC_FP8TOK:
      return orc_dec_e4m3(((const uint8_t *)x->data)[r * K + k]);
    case ORC_MXFP8:
      return orc_dec_e4m3(((const uint8_t *)x->data)[r * K + k]) *
             orc_dec_e8m0(x->scales[r * (K / 32) + k / 32]);
  }
  return NAN;
}

double orc_rowfactor(const orc_operand *x, int64_t r) {
  if (x->fmt == ORC_NVFP4) return x->tscale;
  if (x->fmt == ORC_FP8TOK) return (double)x->rowscale[r];
  return 1.0;
}

/* -------------------------------------------------------- parallel helper */

typedef struct {
  void (*fn)(void *ctx, int64_t lo, int64_t hi);
  void *ctx;
  int64_t lo, hi;
} orc_job;

static void *orc_job_run(void *p) {
  orc_job *j = (orc_job *)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

/* split [0,n) into contiguous slices, one per thread */
static void orc_parallel(int64_t n, int nthreads, void *ctx,
                         void (*fn)(void *, int64_t, int64_t)) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  orc_job jobs[256];
  int started[256];
  for (int i = 0; i < nthreads; i++) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].lo = n * i / nthreads;
    jobs[i].hi = n * (i + 1) / nthreads;
    started[i] = pthread_create(&th[i], NULL, orc_job_run, &jobs[i]) == 0;
    if (!started[i]) orc_job_run(&jobs[i]);
  }
  for (int i = 0; i < nthreads; i++)
    if (started[i]) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------- GEMM */

typedef struct {
  const orc_operand *A, *W;
  const int64_t *m, *n;
  int64_t N; /* for full mode: points enumerated row-major */
  double *C, *B;
} orc_gemm_ctx;

static void orc_gemm_one(const orc_operand *A, const orc_operand *W, int64_t m,
                         int64_t n, double *c, double *b) {
  /* C[m,n] = f_A(m) f_W(n) sum_k a(m,k) w(n,k); B the same with |.| */
  double s = 0.0, sa = 0.0;
  for (int64_t k = 0; k < A->K; k++) {
    double p = orc_elem(A, m, k) * orc_elem(W, n, k);
    s += p;
    sa += fabs(p);
  }
  double f = orc_rowfactor(A, m) * orc_rowfactor(W, n);
  *c = f * s;
  *b = fabs(f) * sa;
}

static void orc_gemm_points_range(void *p, int64_t lo, int64_t hi) {
  orc_gemm_ctx *c = (orc_gemm_ctx *)p;
  for (int64_t i = lo; i < hi; i++)
    orc_gemm_one(c->A, c->W, c->m[i], c->n[i], &c->C[i], &c->B[i]);
}

static void orc_gemm_full_range(void *p, int64_t lo, int64_t hi) {
  orc_gemm_ctx *c = (orc_gemm_ctx *)p;
  for (int64_t i = lo; i < hi; i++)
    orc_gemm_one(c->A, c->W, i / c->N, i % c->N, &c->C[i], &c->B[i]);
}

static int orc_operand_ok(const orc_operand *x) {
  if (!x || !x->data || x->R < 0 || x->K <= 0) return 0;
  if (x->fmt == ORC_NVFP4) return x->scales && x->K % 16 == 0;
  if (x->fmt == ORC_MXFP8) return x->scales && x->K % 32 == 0;
  if (x->fmt == ORC_FP8TOK) return x->rowscale != NULL;
  return x->fmt == ORC_BF16;
}

int orc_gemm_points(const orc_operand *A, const orc_operand *W,
                    const int64_t *m, const int64_t *n, int64_t npts,
                    double *C, double *B, int nthreads) {
  if (!orc_operand_ok(A) || !orc_operand_ok(W) || A->K != W->K) return -1;
  if (npts < 0 || (npts > 0 && (!m || !n || !C || !B))) return -1;
  for (int64_t i = 0; i < npts; i++)
    if (m[i] < 0 || m[i] >= A->R || n[i] < 0 || n[i] >= W->R) return -1;
  orc_gemm_ctx c = {A, W, m, n, 0, C, B};
  orc_parallel(npts, nthreads, &c, orc_gemm_points_range);
  return 0;
}

int orc_gemm_full(const orc_operand *A, const orc_operand *W, double *C,
                  double *B, int nthreads) {
  if (!orc_operand_ok(A) || !orc_operand_ok(W) || A->K != W->K) return -1;
  if (!C || !B) return -1;
  orc_gemm_ctx c = {A, W, NULL, NULL, W->R, C, B};
  orc_parallel(A->R * W->R, nthreads, &c, orc_gemm_full_range);
  return 0;
}

/* ------------------------------------------- exact-FP8 route, emulated */

uint32_t orc_fp8route_convert_word(uint32_t q) {
  /* hardware::exec docs, module description: keep each byte's sign bit and
     move its three magnitude bits down by two, turning an E2M1 code held in
     bits 7..4 into an E4M3 byte whose value is the code's value times 2^-6 */
  return (q & 0x80808080u) | ((q & 0x70707070u) >> 2);
}

/* E4M3 value of element k of an NVFP4 row, reached through the bit identity */
static double orc_fp8route_elem(const uint8_t *q, int64_t k) {
  uint8_t byte = q[k / 2];
  uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  uint32_t word = (uint32_t)code << 4; /* the code in bits 7..4 of byte 0 */
  uint32_t conv = orc_fp8route_convert_word(word);
  return orc_dec_e4m3((uint8_t)(conv & 0xFF));
}

float orc_fp8route_w4a4_point(const uint8_t *aq, const uint8_t *as,
                              const uint8_t *wq, const uint8_t *ws, int64_t K) {
  float acc = 0.0f;
  for (int64_t g = 0; g < K / 16; g++) {
    double p = 0.0; /* group partial of converted operands */
    for (int64_t k = 16 * g; k < 16 * g + 16; k++)
      p += orc_fp8route_elem(aq, k) * orc_fp8route_elem(wq, k);
    float pg = (float)p;
    /* the folded 2^6 per operand: each decoded group scale times 64, in FP32 */
    float ca = (float)(64.0 * orc_dec_e4m3(as[g]));
    float cw = (float)(64.0 * orc_dec_e4m3(ws[g]));
    float c = ca * cw;
    acc = fmaf(c, pg, acc);
  }
  return acc;
}

float orc_fp8route_w4a8_point(const uint8_t *a8, const uint8_t *wq,
                              const uint8_t *ws, int64_t K) {
  float acc = 0.0f;
  for (int64_t g = 0; g < K / 16; g++) {
    double p = 0.0;
    for (int64_t k = 16 * g; k < 16 * g + 16; k++)
      p += orc_dec_e4m3(a8[k]) * orc_fp8route_elem(wq, k);
    float pg = (float)p;
    float c = (float)(64.0 * orc_dec_e4m3(ws[g]));
    acc = fmaf(c, pg, acc);
  }
  return acc;
}

void orc_fp8route_w4a4_rows(const uint8_t *aq, const uint8_t *as,
                            const uint8_t *wq, const uint8_t *ws, int64_t K,
                            int64_t nrows, float *out) {
  for (int64_t i = 0; i < nrows; i++)
    out[i] = orc_fp8route_w4a4_point(aq + i * (K / 2), as + i * (K / 16),
                                     wq + i * (K / 2), ws + i * (K / 16), K);
}

void orc_fp8route_w4a8_rows(const uint8_t *a8, const uint8_t *wq,
                            const uint8_t *ws, int64_t K, int64_t nrows, float *out) {
  for (int64_t i = 0; i < nrows; i++)
    out[i] = orc_fp8route_w4a8_point(a8 + i * K, wq + i * (K / 2), ws + i * (K / 16), K);
}

typedef struct {
  const uint8_t *aq, *as, *wq, *ws;
  int64_t K;
  const int64_t *m, *n;
  float *out;
} orc_route_ctx;

static void orc_route_points_range(void *p, int64_t lo, int64_t hi) {
  orc_route_ctx *c = (orc_route_ctx *)p;
  const int64_t K = c->K;
  for (int64_t i = lo; i < hi; i++)
    c->out[i] = orc_fp8route_w4a4_point(c->aq + c->m[i] * (K / 2), c->as + c->m[i] * (K / 16),
                                        c->wq + c->n[i] * (K / 2), c->ws + c->n[i] * (K / 16), K);
}

int orc_fp8route_w4a4_points(const uint8_t *aq, const uint8_t *as, const uint8_t *wq,
                             const uint8_t *ws, int64_t M, int64_t N, int64_t K,
                             const int64_t *m, const int64_t *n, int64_t npts, float *out,
                             int nthreads) {
  if (!aq || !as || !wq || !ws || K <= 0 || K % 16 || npts < 0) return -1;
  if (npts > 0 && (!m || !n || !out)) return -1;
  for (int64_t i = 0; i < npts; i++)
    if (m[i] < 0 || m[i] >= M || n[i] < 0 || n[i] >= N) return -1;
  orc_route_ctx c = {aq, as, wq, ws, K, m, n, out};
  orc_parallel(npts, nthreads, &c, orc_route_points_range);
  return 0;
}

/* --------------------------------------------------------------- encoders */

uint8_t orc_enc_e4m3_rne_sat(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t s = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return s | 0x7E; /* saturate to the largest finite value */
  if (a == 0.0) return s;
  int x;
  frexp(a, &x);
  int e = x - 1;          /* floor(log2 a) */
  if (e < -6) e = -6;     /* below the normal range the step is fixed */
  double quantum = ldexp(1.0, e - 3);
  double r = rint(a / quantum) * quantum; /* ties to even (default mode) */
  if (r >= 448.0) return s | 0x7E;
  if (r == 0.0) return s;
  if (r < ldexp(1.0, -6)) { /* subnormal: r = m * 2^-9 */
    int m = (int)(r / ldexp(1.0, -9));
    return s | (uint8_t)m;
  }
  frexp(r, &x);
  int er = x - 1;
  int m = (int)((r / ldexp(1.0, er) - 1.0) * 8.0);
  return s | (uint8_t)((er + 7) << 3) | (uint8_t)m;
}

void orc_mxq(const float *v, int64_t n, uint8_t *codes, uint8_t *scales) {
  for (int64_t b = 0; b < n / 32; b++) {
    double amax = 0.0;
    for (int64_t i = 0; i < 32; i++) {
      double a = fabs((double)v[32 * b + i]);
      if (a > amax) amax = a;
    }
    if (amax == 0.0) {
      scales[b] = 0;
      for (int64_t i = 0; i < 32; i++) codes[32 * b + i] = 0;
      continue;
    }
    int x;
    frexp(amax, &x);
    int X = (x - 1) - 8; /* floor(log2 amax) minus the E4M3 max exponent */
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    scales[b] = (uint8_t)(X + 127);
    for (int64_t i = 0; i < 32; i++)
      codes[32 * b + i] = orc_enc_e4m3_rne_sat(ldexp((double)v[32 * b + i], -X));
  }
}

uint16_t orc_bf16_rne(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return s;
  int x;
  frexp(a, &x);
  int e = x - 1;
  if (e < -126) e = -126; /* subnormal BF16 step is 2^-133 */
  double quantum = ldexp(1.0, e - 7);
  double r = rint(a / quantum) * quantum;
  if (r >= ldexp(1.0, 128)) return s | 0x7F80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return s | (uint16_t)(bits >> 16);
}

/* -------------------------------------------------------------------- MoE */

static double orc_mx_elem(const uint8_t *q, const uint8_t *s, int64_t row,
                          int64_t K, int64_t k) {
  return orc_dec_e4m3(q[row * K + k]) * orc_dec_e8m0(s[row * (K / 32) + k / 32]);
}

void orc_moe_gateup(const uint8_t *xq, const uint8_t *xs, int64_t t, int64_t e,
                    const uint8_t *w13q, const uint8_t *w13s, int64_t H, int64_t I,
                    double *g, double *u, double *bg, double *bu) {
  for (int64_t i = 0; i < I; i++) {
    int64_t rg = e * 2 * I + i, ru = e * 2 * I + I + i;
    double sg = 0, su = 0, ag = 0, au = 0;
    for (int64_t k = 0; k < H; k++) {
      double x = orc_mx_elem(xq, xs, t, H, k);
      double pg = x * orc_mx_elem(w13q, w13s, rg, H, k);
      double pu = x * orc_mx_elem(w13q, w13s, ru, H, k);
      sg += pg;
      su += pu;
      ag += fabs(pg);
      au += fabs(pu);
    }
    g[i] = sg;
    u[i] = su;
    if (bg) bg[i] = ag;
    if (bu) bu[i] = au;
  }
}

void orc_moe_glu_requant(const double *g, const double *u, int64_t I,
                         uint8_t *hq, uint8_t *hs) {
  float *h = (float *)malloc(sizeof(float) * (size_t)I);
  for (int64_t i = 0; i < I; i++) {
    double silu = g[i] / (1.0 + exp(-g[i]));
    h[i] = (float)(silu * u[i]); /* the requant decision is taken in FP32 */
  }
  orc_mxq(h, I, hq, hs);
  free(h);
}

void orc_moe_down(const uint8_t *hq, const uint8_t *hs, int64_t e,
                  const uint8_t *w2q, const uint8_t *w2s, int64_t H, int64_t I,
                  double *y, double *by) {
  for (int64_t n = 0; n < H; n++) {
    double s = 0, a = 0;
    for (int64_t i = 0; i < I; i++) {
      double p = orc_dec_e4m3(hq[i]) * orc_dec_e8m0(hs[i / 32]) *
                 orc_mx_elem(w2q, w2s, e * H + n, I, i);
      s += p;
      a += fabs(p);
    }
    y[n] = s;
    if (by) by[n] = a;
  }
}

typedef struct {
  const uint8_t *xq, *xs;
  const int32_t *ids;
  const float *tw;
  int64_t T, H, I, E, topk;
  const uint8_t *w13q, *w13s, *w2q, *w2s;
  const int64_t *tokens;
  double *out, *bound;
} orc_moe_ctx;

static void orc_moe_range(void *p, int64_t lo, int64_t hi) {
  orc_moe_ctx *c = (orc_moe_ctx *)p;
  const int64_t H = c->H, I = c->I;
  double *g = (double *)malloc(sizeof(double) * (size_t)I);
  double *u = (double *)malloc(sizeof(double) * (size_t)I);
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  double *by = (double *)malloc(sizeof(double) * (size_t)H);
  uint8_t *hq = (uint8_t *)malloc((size_t)I);
  uint8_t *hs = (uint8_t *)malloc((size_t)(I / 32));
  for (int64_t ti = lo; ti < hi; ti++) {
    int64_t t = c->tokens[ti];
    double *o = c->out + ti * H, *b = c->bound + ti * H;
    for (int64_t n = 0; n < H; n++) o[n] = b[n] = 0.0;
    for (int64_t j = 0; j < c->topk; j++) {
      int64_t e = c->ids[t * c->topk + j];
      double w = (double)c->tw[t * c->topk + j];
      orc_moe_gateup(c->xq, c->xs, t, e, c->w13q, c->w13s, H, I, g, u, NULL, NULL);
      orc_moe_glu_requant(g, u, I, hq, hs);
      orc_moe_down(hq, hs, e, c->w2q, c->w2s, H, I, y, by);
      for (int64_t n = 0; n < H; n++) {
        o[n] += w * y[n];
        b[n] += fabs(w) * by[n];
      }
    }
  }
  free(g); free(u); free(y); free(by); free(hq); free(hs);
}

int orc_moe_tokens(const uint8_t *xq, const uint8_t *xs, const int32_t *ids,
                   const float *tw, int64_t T, int64_t H, int64_t I, int64_t E,
                   int64_t topk, const uint8_t *w13q, const uint8_t *w13s,
                   const uint8_t *w2q, const uint8_t *w2s,
                   const int64_t *tokens, int64_t ntok,
                   double *out, double *bound, int nthreads) {
  if (!xq || !xs || !ids || !tw || !w13q || !w13s || !w2q || !w2s) return -1;
  if (H % 32 || I % 32 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return -1;
  if (ntok < 0 || (ntok > 0 && (!tokens || !out || !bound))) return -1;
  for (int64_t i = 0; i < ntok; i++) {
    if (tokens[i] < 0 || tokens[i] >= T) return -1;
    for (int64_t j = 0; j < topk; j++) {
      int32_t e = ids[tokens[i] * topk + j];
      if (e < 0 || e >= E) return -1;
    }
  }
  orc_moe_ctx c = {xq, xs, ids, tw, T, H, I, E, topk,
                   w13q, w13s, w2q, w2s, tokens, out, bound};
  orc_parallel(ntok, nthreads, &c, orc_moe_range);
  return 0;
}

/* ------------------------------------------------------------- NVFP4 MoE */
/* The GLU MoE of the functions above with NVFP4 operands: x with one FP32
 * tensor scale Sx, each expert's w13 and w2 with one FP32 tensor scale per
 * expert, and h re-quantised to NVFP4 under a tensor scale Sh that the caller
 * fixes.  Values decode exactly to FP64 and every sum runs in ascending k. */

static double orc_nv_elem(const uint8_t *q, const uint8_t *s, int64_t row, int64_t K,
                          int64_t k) {
  uint8_t byte = q[row * (K / 2) + k / 2];
  uint8_t code = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
  return orc_dec_e2m1(code) * orc_dec_e4m3(s[row * (K / 16) + k / 16]);
}

/* FP32 value -> E2M1 code (sign in bit 3): the nearest of the eight
 * magnitudes, a tie going to the code with a zero low bit; magnitudes above 6
 * give 6; NaN gives 0. */
uint8_t orc_enc_e2m1_rne_sat(float v) {
  if (isnan(v)) return 0;
  uint8_t sgn = signbit(v) ? 8 : 0;
  double a = fabs((double)v);
  if (a >= 6.0) return sgn | 7; /* saturate (distances to 4 and 6 tie for huge a) */
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 8; c++) {
    double d = fabs(a - orc_dec_e2m1((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return sgn | (uint8_t)best;
}

/* NVFP4 quantisation of n FP32 values (n % 16 == 0) under tensor scale S,
 * taken in FP32: per group of 16, scale byte = E4M3(amax / 6 / S) (nearest
 * even, saturating), then code = E2M1(v / (e4m3(scale) * S)); a zero scale
 * gives zero codes.  Codes are packed two per byte, element 2j in the low
 * nibble. */
void orc_nvq(const float *v, int64_t n, float S, uint8_t *codes, uint8_t *scales) {
  for (int64_t g = 0; g < n / 16; g++) {
    float amax = 0.0f;
    for (int64_t i = 0; i < 16; i++) {
      float a = fabsf(v[16 * g + i]);
      if (a > amax) amax = a;
    }
    float sv = amax / 6.0f / S;
    uint8_t sb = orc_enc_e4m3_rne_sat((double)sv);
    scales[g] = sb;
    float d = (float)orc_dec_e4m3(sb) * S;
    for (int64_t i = 0; i < 16; i += 2) {
      uint8_t c0 = 0, c1 = 0;
      if ((sb & 0x7F) != 0) {
        c0 = orc_enc_e2m1_rne_sat(v[16 * g + i] / d);
        c1 = orc_enc_e2m1_rne_sat(v[16 * g + i + 1] / d);
      }
      codes[(16 * g + i) / 2] = (uint8_t)(c0 | (c1 << 4));
    }
  }
}

void orc_moe4_gateup(const uint8_t *xq, const uint8_t *xs, float Sx, int64_t t, int64_t e,
                     const uint8_t *w13q, const uint8_t *w13s, const float *Sw13, int64_t H,
                     int64_t I, double *g, double *u, double *bg, double *bu) {
  const double f = (double)Sx * (double)Sw13[e];
  for (int64_t i = 0; i < I; i++) {
    int64_t rg = e * 2 * I + i, ru = e * 2 * I + I + i;
    double sg = 0, su = 0, ag = 0, au = 0;
    for (int64_t k = 0; k < H; k++) {
      double x = orc_nv_elem(xq, xs, t, H, k);
      double pg = x * orc_nv_elem(w13q, w13s, rg, H, k);
      double pu = x * orc_nv_elem(w13q, w13s, ru, H, k);
      sg += pg;
      su += pu;
      ag += fabs(pg);
      au += fabs(pu);
    }
    g[i] = f * sg;
    u[i] = f * su;
    if (bg) bg[i] = fabs(f) * ag;
    if (bu) bu[i] = fabs(f) * au;
  }
}

void orc_moe4_glu_requant(const double *g, const double *u, int64_t I, float Sh, uint8_t *hq,
                          uint8_t *hs) {
  float *h = (float *)malloc(sizeof(float) * (size_t)I);
  for (int64_t i = 0; i < I; i++) {
    double silu = g[i] / (1.0 + exp(-g[i]));
    h[i] = (float)(silu * u[i]); /* the requant decisions are taken in FP32 */
  }
  orc_nvq(h, I, Sh, hq, hs);
  free(h);
}

void orc_moe4_down(const uint8_t *hq, const uint8_t *hs, float Sh, int64_t e,
                   const uint8_t *w2q, const uint8_t *w2s, const float *Sw2, int64_t H,
                   int64_t I, double *y, double *by) {
  const double f = (double)Sh * (double)Sw2[e];
  for (int64_t n = 0; n < H; n++) {
    double s = 0, a = 0;
    for (int64_t i = 0; i < I; i++) {
      double p = orc_nv_elem(hq, hs, 0, I, i) * orc_nv_elem(w2q, w2s, e * H + n, I, i);
      s += p;
      a += fabs(p);
    }
    y[n] = f * s;
    if (by) by[n] = fabs(f) * a;
  }
}

typedef struct {
  const uint8_t *xq, *xs;
  float Sx, Sh;
  const int32_t *ids;
  const float *tw;
  int64_t T, H, I, E, topk;
  const uint8_t *w13q, *w13s, *w2q, *w2s;
  const float *Sw13, *Sw2;
  const int64_t *tokens;
  double *out, *bound;
} orc_moe4_ctx;

static void orc_moe4_range(void *p, int64_t lo, int64_t hi) {
  orc_moe4_ctx *c = (orc_moe4_ctx *)p;
  const int64_t H = c->H, I = c->I;
  double *g = (double *)malloc(sizeof(double) * (size_t)I);
  double *u = (double *)malloc(sizeof(double) * (size_t)I);
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  double *by = (double *)malloc(sizeof(double) * (size_t)H);
  uint8_t *hq = (uint8_t *)malloc((size_t)(I / 2));
  uint8_t *hs = (uint8_t *)malloc((size_t)(I / 16));
  for (int64_t ti = lo; ti < hi; ti++) {
    int64_t t = c->tokens[ti];
    double *o = c->out + ti * H, *b = c->bound + ti * H;
    for (int64_t n = 0; n < H; n++) o[n] = b[n] = 0.0;
    for (int64_t j = 0; j < c->topk; j++) {
      int64_t e = c->ids[t * c->topk + j];
      double w = (double)c->tw[t * c->topk + j];
      orc_moe4_gateup(c->xq, c->xs, c->Sx, t, e, c->w13q, c->w13s, c->Sw13, H, I, g, u, NULL,
                      NULL);
      orc_moe4_glu_requant(g, u, I, c->Sh, hq, hs);
      orc_moe4_down(hq, hs, c->Sh, e, c->w2q, c->w2s, c->Sw2, H, I, y, by);
      for (int64_t n = 0; n < H; n++) {
        o[n] += w * y[n];
        b[n] += fabs(w) * by[n];
      }
    }
  }
  free(g); free(u); free(y); free(by); free(hq); free(hs);
}

int orc_moe4_tokens(const uint8_t *xq, const uint8_t *xs, float Sx, const int32_t *ids,
                    const float *tw, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                    const uint8_t *w13q, const uint8_t *w13s, const float *Sw13,
                    const uint8_t *w2q, const uint8_t *w2s, const float *Sw2, float Sh,
                    const int64_t *tokens, int64_t ntok, double *out, double *bound,
                    int nthreads) {
  if (!xq || !xs || !ids || !tw || !w13q || !w13s || !Sw13 || !w2q || !w2s || !Sw2) return -1;
  if (H % 16 || I % 16 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return -1;
  if (ntok < 0 || (ntok > 0 && (!tokens || !out || !bound))) return -1;
  for (int64_t i = 0; i < ntok; i++) {
    if (tokens[i] < 0 || tokens[i] >= T) return -1;
    for (int64_t j = 0; j < topk; j++) {
      int32_t e = ids[tokens[i] * topk + j];
      if (e < 0 || e >= E) return -1;
    }
  }
  orc_moe4_ctx c = {xq, xs, Sx, Sh, ids, tw, T, H, I, E, topk,
                    w13q, w13s, w2q, w2s, Sw13, Sw2, tokens, out, bound};
  orc_parallel(ntok, nthreads, &c, orc_moe4_range);
  return 0;
}

/* --------------------------------------------------------- top-k routing */
/* Routing of the MoE configuration (softmax of the router logits, top k):
 * per token, p_e = exp(l_e - max l) / sum_e' exp(l_e' - max l) in FP64; the k
 * experts of largest p in descending order, equal p going to the lower id;
 * weights the probabilities themselves (not renormalised), rounded to FP32.
 * The order is taken on the logits, which gives the order of the exact
 * probabilities (the softmax is increasing in the logit) without the ties an
 * FP64 exp could create between distinct logits. */
int orc_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids,
                     float *w) {
  if (!logits || !ids || !w || T < 0 || E <= 0 || topk <= 0 || topk > E) return -1;
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  unsigned char *used = (unsigned char *)malloc((size_t)E);
  for (int64_t t = 0; t < T; t++) {
    const float *l = logits + t * E;
    double m = -INFINITY, s = 0.0;
    for (int64_t e = 0; e < E; e++) if ((double)l[e] > m) m = (double)l[e];
    for (int64_t e = 0; e < E; e++) {
      p[e] = exp((double)l[e] - m);
      s += p[e];
      used[e] = 0;
    }
    for (int64_t j = 0; j < topk; j++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++)
        if (!used[e] && (best < 0 || l[e] > l[best])) best = e;
      used[best] = 1;
      ids[t * topk + j] = (int32_t)best;
      w[t * topk + j] = (float)(p[best] / s);
    }
  }
  free(p);
  free(used);
  return 0;
}
