/*
 * oracle.h -- plain FP64 CPU oracle for the block-scaled TN GEMM hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
 * Python binding) includes, links or calls this code.  Only the tests, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
 * code, header, table or constant generator with the GPU path.
 *
 * What it computes (all in FP64, each product formed exactly, summed in
 * ascending k):
 *
 *   C[m,n] = f_A(m) * f_W(n) * sum_k a(m,k) * w(n,k)
 *   B[m,n] = |f_A(m) * f_W(n)| * sum_k |a(m,k) * w(n,k)|
 *
 * where a(.,.) / w(.,.) are the decoded element values including their block
 * scale, and f_X(r) the per-row factor (FP32 tensor scale of an NVFP4
 * operand, or the per-token FP32 scale of an FP8 activation).  The formats
 * are those the hardware::exec module documentation (metrale_circuit) lists
 * for weight-reading nodes: BF16, NVFP4 (E2M1 codes, one E4M3 scale per 16
 * K-elements, one FP32 tensor scale), FP8 E4M3 with a per-token scale, and
 * MXFP8 (E4M3 codes, one E8M0 scale per 32 K-elements).
 *
 * Parity status of each function is stated at its declaration.
 */
#ifndef BSP_ORACLE_H
#define BSP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Operand formats (oracle-private numbering). */
enum { ORC_BF16 = 0, ORC_NVFP4 = 1, ORC_FP8TOK = 2, ORC_MXFP8 = 3 };

typedef struct {
  int fmt;
  const void *data;       /* BF16: uint16 [R,K]; NVFP4: uint8 [R,K/2] (element 2i low nibble);
                             FP8TOK / MXFP8: uint8 [R,K] E4M3 bytes */
  const uint8_t *scales;  /* NVFP4: E4M3 [R,K/16]; MXFP8: E8M0 [R,K/32]; else NULL */
  const float *rowscale;  /* FP8TOK: FP32 [R]; else NULL */
  double tscale;          /* NVFP4: the FP32 tensor scale value; else 1 */
  int64_t R, K;
} orc_operand;

/* --- element decoders (pinned: closed forms + exhaustive tables in tests) --- */
double orc_dec_bf16(uint16_t u);
double orc_dec_e2m1(uint8_t code);   /* low 4 bits used */
double orc_dec_e4m3(uint8_t b);      /* OCP E4M3-FN; NaN for 0x7F/0xFF */
double orc_dec_e8m0(uint8_t x);      /* 2^(x-127); NaN for 0xFF */

/* decoded element (r,k) of an operand, block scale included, row factor not */
double orc_elem(const orc_operand *x, int64_t r, int64_t k);
/* the per-row factor f_X(r) */
double orc_rowfactor(const orc_operand *x, int64_t r);

/* C and B at the listed points (m[i], n[i]).  nthreads <= 0 means 1.
   Returns 0, or -1 on bad arguments.  Pinned (hand cases, brute force,
   exact-sum regime, invariants). */
int orc_gemm_points(const orc_operand *A, const orc_operand *W,
                    const int64_t *m, const int64_t *n, int64_t npts,
                    double *C, double *B, int nthreads);
/* all M x N points, row-major [M,N] */
int orc_gemm_full(const orc_operand *A, const orc_operand *W,
                  double *C, double *B, int nthreads);

/* --- the exact-FP8 route of the hardware::exec docs, emulated bit by bit ---
   E2M1 code (bits 7..4 of a byte) -> E4M3 byte via the pages' mask-and-shift
   identity; a 16-element group partial formed in FP32; the two group scales
   decoded, multiplied by 64 each, multiplied together in FP32; one FP32 fused
   multiply-add per group into the accumulator, groups ascending.  Returns the
   FP32 accumulator before the tensor scales.  Pinned against orc_gemm_points
   by exhaustive search over codes and scales (the pages' equivalence claim). */
uint32_t orc_fp8route_convert_word(uint32_t q);   /* four codes in bits 7..4 of each byte */
float orc_fp8route_w4a4_point(const uint8_t *aq, const uint8_t *as,
                              const uint8_t *wq, const uint8_t *ws, int64_t K);
float orc_fp8route_w4a8_point(const uint8_t *a8, const uint8_t *wq,
                              const uint8_t *ws, int64_t K);
/* row i of A against row i of W, for i < nrows (brute-force sweeps) */
void orc_fp8route_w4a4_rows(const uint8_t *aq, const uint8_t *as,
                            const uint8_t *wq, const uint8_t *ws, int64_t K,
                            int64_t nrows, float *out);
void orc_fp8route_w4a8_rows(const uint8_t *a8, const uint8_t *wq,
                            const uint8_t *ws, int64_t K, int64_t nrows, float *out);

/* the emulated route at points: row m[i] of A ([M,K/2] codes, [M,K/16]
   scales) against row n[i] of W; returns 0, or -1 on bad arguments */
int orc_fp8route_w4a4_points(const uint8_t *aq, const uint8_t *as, const uint8_t *wq,
                             const uint8_t *ws, int64_t M, int64_t N, int64_t K,
                             const int64_t *m, const int64_t *n, int64_t npts, float *out,
                             int nthreads);

/* --- encoders used by the MoE requant step (and pinned by round trips) --- */
/* round-to-nearest-even onto the E4M3-FN grid, saturating at +-448 */
uint8_t orc_enc_e4m3_rne_sat(double v);
/* MXFP8 block quantiser (OCP MX rule, E4M3 elements, E8M0 shared scale per
   32): X = floor(log2(amax)) - 8 clamped to [-127,127]; amax == 0 gives
   scale byte 0 and zero codes.  n must be a multiple of 32. */
void orc_mxq(const float *v, int64_t n, uint8_t *codes, uint8_t *scales);

/* --- MXFP8 grouped MoE GLU (configuration: E experts, top-k routing) ---
   Stage functions and the end-to-end result.  Rows of w13 are [gate; up]:
   w13 is [E, 2I, H] (rows [0,I) gate, [I,2I) up), w2 is [E, H, I]. */
/* g[i], u[i] for token t through expert e (FP64), and the matching |.| sums */
void orc_moe_gateup(const uint8_t *xq, const uint8_t *xs, int64_t t, int64_t e,
                    const uint8_t *w13q, const uint8_t *w13s, int64_t H, int64_t I,
                    double *g, double *u, double *bg, double *bu);
/* h = silu(g) * u in FP64, rounded to FP32 (the precision in which the
   quantisation decision is taken), then MXFP8-quantised.  Parity of the
   requant step is checked stage-wise (several codes can be correct where h
   lies on a rounding boundary). */
void orc_moe_glu_requant(const double *g, const double *u, int64_t I,
                         uint8_t *hq, uint8_t *hs);
/* y[n] = sum_i dec(hq)_i * dec(w2[e][n])_i, and its |.| sum */
void orc_moe_down(const uint8_t *hq, const uint8_t *hs, int64_t e,
                  const uint8_t *w2q, const uint8_t *w2s, int64_t H, int64_t I,
                  double *y, double *by);
/* End to end for the listed tokens: out[t,:] (FP64) and bound[t,:].
   Uses the stages above: gate/up in FP64, h rounded to FP32, requantised,
   down in FP64, combine over slots j ascending with FP32 routing weights. */
int orc_moe_tokens(const uint8_t *xq, const uint8_t *xs, const int32_t *ids,
                   const float *tw, int64_t T, int64_t H, int64_t I, int64_t E,
                   int64_t topk, const uint8_t *w13q, const uint8_t *w13s,
                   const uint8_t *w2q, const uint8_t *w2s,
                   const int64_t *tokens, int64_t ntok,
                   double *out, double *bound, int nthreads);

/* round-to-nearest-even of an FP64 value to BF16 bits (no double rounding) */
uint16_t orc_bf16_rne(double v);

/* --- NVFP4 grouped MoE GLU: the MoE above with NVFP4 operands ---
   x: codes [T,H/2] (element 2j in the low nibble), E4M3 scales [T,H/16],
   FP32 tensor scale Sx.  w13 [E,2I,H/2] + [E,2I,H/16], one FP32 tensor scale
   per expert Sw13[E]; w2 [E,H,I/2] + [E,H,I/16], Sw2[E].  h is re-quantised
   to NVFP4 under the caller's tensor scale Sh. */
/* FP32 -> E2M1 code: nearest magnitude of {0,.5,1,1.5,2,3,4,6}, ties to the
   code with a zero low bit, saturating at 6, sign in bit 3; NaN -> 0 */
uint8_t orc_enc_e2m1_rne_sat(float v);
/* NVFP4 quantiser taken in FP32: per 16, scale = E4M3(amax / 6 / S), codes =
   E2M1(v / (e4m3(scale) * S)); a zero scale gives zero codes.  n % 16 == 0;
   codes packed two per byte. */
void orc_nvq(const float *v, int64_t n, float S, uint8_t *codes, uint8_t *scales);
/* g = Sx Sw13[e] sum_k x_k w13[e][i]_k, u likewise for row I+i, and bounds */
void orc_moe4_gateup(const uint8_t *xq, const uint8_t *xs, float Sx, int64_t t, int64_t e,
                     const uint8_t *w13q, const uint8_t *w13s, const float *Sw13, int64_t H,
                     int64_t I, double *g, double *u, double *bg, double *bu);
/* h = silu(g) * u in FP64, rounded to FP32, then orc_nvq under Sh */
void orc_moe4_glu_requant(const double *g, const double *u, int64_t I, float Sh, uint8_t *hq,
                          uint8_t *hs);
/* y[n] = Sh Sw2[e] sum_i dec(hq)_i dec(w2[e][n])_i, and its bound */
void orc_moe4_down(const uint8_t *hq, const uint8_t *hs, float Sh, int64_t e,
                   const uint8_t *w2q, const uint8_t *w2s, const float *Sw2, int64_t H,
                   int64_t I, double *y, double *by);
/* end to end for the listed tokens, as orc_moe_tokens */
int orc_moe4_tokens(const uint8_t *xq, const uint8_t *xs, float Sx, const int32_t *ids,
                    const float *tw, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
                    const uint8_t *w13q, const uint8_t *w13s, const float *Sw13,
                    const uint8_t *w2q, const uint8_t *w2s, const float *Sw2, float Sh,
                    const int64_t *tokens, int64_t ntok, double *out, double *bound,
                    int nthreads);

/* --- top-k softmax routing of the MoE configuration ---
   Per token t: p = softmax(logits[t,:]) in FP64; the topk experts of largest
   p, descending, equal p to the lower id (ordered on the logits, which is the
   order of the exact probabilities); w = p rounded to FP32 (not
   renormalised).  logits [T,E] finite FP32; ids, w [T,topk]. */
int orc_topk_softmax(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *ids,
                     float *w);

#ifdef __cplusplus
}
#endif
#endif
