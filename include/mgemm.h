/*
 * mgemm.h -- C ABI of the MI355X (gfx950) block-scaled TN GEMM library.
 *
 * One operation, several declared formats:
 *
 *     C[M,N] = A[M,K] . W[N,K]^T      (FP32 accumulation, BF16 output)
 *
 * All operands are K-contiguous ("TN"): A is [M,K] row-major, W is [N,K]
 * row-major, C is [M,N] row-major.  The declared formats and how each one
 * executes follow the metrale_circuit "hardware::exec" module documentation
 * (module description; entries exec_of, fp4_fallback, kind_of, node_exec,
 * pair_name): the activation format picks the matrix instruction, NVFP4
 * operands on a device without an NVFP4 block-scale MMA go through the exact
 * E2M1 -> E4M3 conversion onto the FP8 MMA with the group scales applied in
 * FP32 per K=16 step, and a pair with no native or exact path has no path --
 * it is never re-run at a wider format.
 *
 * Storage formats
 *   BF16        uint16 bits, [R,K].
 *   NVFP4       codes uint8 [R,K/2], element 2i in the LOW nibble of byte i,
 *               element 2i+1 in the high nibble (E2M1: sign bit 3, exponent
 *               bits 2..1, mantissa bit 0); scales uint8 [R,K/16] E4M3-FN, one
 *               per 16 consecutive K-elements; one FP32 tensor scale S (a
 *               DEVICE pointer to one float).  Value = e2m1 * e4m3 * S.
 *   FP8 token   E4M3-FN bytes [M,K] and one FP32 scale per row (device
 *               pointer, [M]).  Value = e4m3 * s[m].
 *   MXFP8       E4M3-FN bytes [R,K] and E8M0 bytes [R,K/32] (2^(x-127)).
 *
 * Calling conventions (every GEMM entry point)
 *   - Pointers are DEVICE pointers of the current HIP device unless stated;
 *     the caller owns every buffer.  The library allocates nothing for the
 *     GEMMs and keeps no state between calls; calls are reentrant.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  C is fully overwritten (no beta).
 *   - out_f32 = 0: C is BF16 (round to nearest even from the FP32 result).
 *     out_f32 = 1: C is FP32 (the accumulator after the global scales).
 *   - K must be a positive multiple of 32; M, N must be positive.  Base
 *     pointers must be 16-byte aligned.
 *   - Data values are not validated (a NaN scale byte gives NaN results).
 *
 * Return codes: 0 on success, a negative MGEMM_ERR_* otherwise;
 * mgemm_status_string() names them.  Argument errors are detected on the
 * host before anything is enqueued.
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* declared storage formats */
enum {
  MGEMM_FMT_BF16 = 0,
  MGEMM_FMT_NVFP4 = 1,
  MGEMM_FMT_FP8_E4M3_TOKEN = 2,
  MGEMM_FMT_MXFP8 = 3
};

/* execution kind of one (weight, activation) pair on a device */
enum { MGEMM_EXEC_NATIVE = 0, MGEMM_EXEC_FP8_EXACT = 1, MGEMM_EXEC_NOPATH = 2 };

/* the matrix instruction that carries the declared formats */
enum {
  MGEMM_MMA_NONE = 0,
  MGEMM_MMA_BF16 = 1,        /* v_mfma_f32_32x32x16_bf16 */
  MGEMM_MMA_FP8 = 2,         /* v_mfma_f32_32x32x16_fp8_fp8, one K=16 group each */
  MGEMM_MMA_MX_F8F6F4 = 3    /* v_mfma_scale_f32_32x32x64_f8f6f4, E8M0 per 32 */
};

/* why a pair runs the way it does (0 = native) */
enum {
  MGEMM_REASON_NONE = 0,
  MGEMM_REASON_NO_INSTRUCTION = 1,        /* no instruction can carry the pair exactly */
  MGEMM_REASON_NO_KERNEL = 2,             /* the library compiles no kernel for the pair */
  MGEMM_REASON_NO_NVFP4_BLOCKSCALE_MMA = 3, /* the FP4 MMA here is MX-scaled only */
  MGEMM_REASON_NO_SINGLE_MMA = 4,         /* NVFP4 weights under FP8 activations */
  MGEMM_REASON_UNSUPPORTED_DEVICE = 5     /* not a gfx950 device */
};

typedef struct {
  int kind;   /* MGEMM_EXEC_* */
  int mma;    /* MGEMM_MMA_* */
  int reason; /* MGEMM_REASON_* */
} mgemm_plan_t;

/* status codes */
enum {
  MGEMM_OK = 0,
  MGEMM_ERR_INVALID_ARG = -1, /* NULL pointer, bad enum, misaligned pointer */
  MGEMM_ERR_SHAPE = -2,       /* M/N/K not positive, K % 32 != 0, size overflow */
  MGEMM_ERR_NOPATH = -3,      /* the plan for this pair on this device is NOPATH */
  MGEMM_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
  MGEMM_ERR_HIP = -5          /* a HIP runtime call or launch failed */
};

/* --------------------------------------------------------------- planning */

/* How device `device` executes a node with weight format w_fmt under
   activation format a_fmt (hardware::exec docs: exec_of, fp4_fallback,
   kind_of, node_exec).  Host only; enqueues nothing.  On gfx950:
     BF16 x BF16   -> NATIVE, BF16 MMA
     NVFP4 w, BF16 a -> NATIVE, BF16 MMA (weights widened in registers, exact)
     NVFP4 w, FP8 a  -> FP8_EXACT, FP8 MMA (reason NO_SINGLE_MMA)
     NVFP4 w, NVFP4 a -> FP8_EXACT, FP8 MMA (reason NO_NVFP4_BLOCKSCALE_MMA)
     MXFP8 x MXFP8 -> NATIVE, MX f8f6f4 MMA
     anything else -> NOPATH.  Any other device -> NOPATH (UNSUPPORTED_DEVICE).
   Returns 0, MGEMM_ERR_INVALID_ARG (bad enum / NULL out), MGEMM_ERR_HIP. */
int mgemm_plan(int device, int w_fmt, int a_fmt, mgemm_plan_t *out);

/* The same decision for a named architecture (e.g. "gfx950:sramecc+:xnack-");
   needs no GPU.  Only the part before the first ':' is compared. */
int mgemm_plan_arch(const char *gcn_arch, int w_fmt, int a_fmt, mgemm_plan_t *out);

/* The declared pair as text, "W<bits>A<bits>" (hardware::exec docs:
   pair_name): BF16 = 16, NVFP4 = 4, FP8 = 8, MXFP8 = 8, e.g. "W4A16".
   Writes a NUL-terminated string into buf (host memory, len bytes).
   Returns the string length, or MGEMM_ERR_INVALID_ARG. */
int mgemm_pair_name(int w_fmt, int a_fmt, char *buf, size_t len);

/* ------------------------------------------------------------------ GEMMs */

/* W16A16: C = A . W^T with BF16 A [M,K] and W [N,K] on the BF16 MFMA,
   FP32 accumulation (the H3 FFN down-projection of RL-Kernel PR #535:
   BF16 MMA tiles, FP32 accumulation, BF16 epilogue).  The grid runs one
   256x256 tile per workgroup (256x128 when an operand reaches 4 GiB) and
   one workgroup per CU; when the tiles fill the last round only in part,
   those tiles are split into K ranges whose
   FP32 partial tiles go to `ws` and a second kernel adds them in range
   order (results are run-to-run bit-identical).  `ws`: device memory of at
   least mgemm_workspace_bytes(MGEMM_OP_BF16, M, N, K, ...) bytes, 16-byte
   aligned, no required contents (size 0: ws may be NULL).  Calls that share
   a workspace must be ordered on one stream.  MGEMM_ERR_WORKSPACE when ws
   is missing, too small or misaligned. */
int mgemm_bf16(const void *A, const void *W, void *C, int64_t M, int64_t N,
               int64_t K, int out_f32, void *ws, size_t ws_bytes, void *stream);

/* W4A16: BF16 activations A [M,K] under NVFP4 weights (Wq [N,K/2],
   Ws [N,K/16], Sw device float*).  Each weight element e2m1*e4m3 is widened
   to BF16 in registers (exact: at most 6 significant bits) and run on the
   BF16 MFMA; Sw is applied in the epilogue (hardware::exec docs, module
   description: BF16 activations take the BF16 MMA with the weight widened).
   Up to 128 tokens take a decode kernel that streams the weight once and
   splits K over workgroups: each writes FP32 partial sums to
   `ws`, and a second kernel adds them in split order (results are
   run-to-run bit-identical).  `ws` is device memory of at least
   mgemm_workspace_bytes(MGEMM_OP_W4A16, M, N, K, ...) bytes, 16-byte
   aligned, with no required contents; more tokens take the tiled kernel and
   need none (size 0: ws may be NULL).  Calls that share a workspace must be
   ordered on one stream.  MGEMM_ERR_WORKSPACE when ws is missing, too small
   or misaligned. */
int mgemm_w4a16(const void *A, const void *Wq, const void *Ws, const float *Sw,
                void *C, int64_t M, int64_t N, int64_t K, int out_f32, void *ws,
                size_t ws_bytes, void *stream);

/* W4A8: FP8 E4M3 activations Aq [M,K] with per-token FP32 scales a_tok [M]
   under NVFP4 weights.  Exact E4M3 route (hardware::exec docs, exec_of):
   weight codes converted by the E2M1 -> E4M3 bit identity, one FP8 MFMA per
   16-element group, the group scale (times 64) applied in FP32 per group,
   a_tok[m] * Sw in the epilogue.  The decode kernel splits K over
   workgroups: each writes FP32 partial sums to `ws`, and a second kernel
   adds them in split order (results are run-to-run bit-identical).  `ws` is
   device memory of at least mgemm_workspace_bytes(MGEMM_OP_W4A8, M, N, K,
   ...) bytes, 16-byte aligned, with no required contents (when the size is
   0, ws may be NULL); a smaller call does not always need less (more than
   64 tokens take a tiled kernel with its own K split), so a shared
   workspace must cover the largest size among its calls.  Calls that share
   a workspace must be ordered on one stream. */
int mgemm_w4a8(const void *Aq, const float *a_tok, const void *Wq, const void *Ws,
               const float *Sw, void *C, int64_t M, int64_t N, int64_t K, int out_f32,
               void *ws, size_t ws_bytes, void *stream);

/* W4A8 without a workspace argument, for callers that cannot allocate
   (code under HIP graph capture, tight serving loops, harnesses that forbid
   hipMalloc).  Computes exactly what mgemm_w4a8 computes, with the same
   kernels and results, but keeps the split-K partials in a fixed device
   buffer of MGEMM_W4A8_NOALLOC_MAX_WS bytes that the library holds on every
   device it runs on, until the process ends.  The call allocates no memory
   (no hipMalloc, hipFree or allocating library routine); its first call on a
   device looks up that device's buffer address.  A call whose
   mgemm_workspace_bytes(MGEMM_OP_W4A8, M, N, K, ...) exceeds the buffer
   returns MGEMM_ERR_WORKSPACE before enqueuing anything (N = 5376, K = 14336
   fits up to M = 128).  The buffer needs no particular contents, but every
   call on one device shares it: calls that overlap on one GPU (on different
   streams, or from several host threads) race and must be ordered by the
   caller.  Other arguments and errors as mgemm_w4a8. */
#define MGEMM_W4A8_NOALLOC_MAX_WS ((size_t)48 << 20)
int mgemm_w4a8_noalloc(const void *Aq, const float *a_tok, const void *Wq, const void *Ws,
                       const float *Sw, void *C, int64_t M, int64_t N, int64_t K, int out_f32,
                       void *stream);

/* W4A4: NVFP4 activations (Aq [M,K/2], As [M,K/16], Sa) under NVFP4 weights.
   Exact E4M3 route (hardware::exec docs, module description and
   fp4_fallback): both operands' codes converted by the E2M1 -> E4M3 bit
   identity, one FP8 MFMA per 16-element group with a zero accumulator, the
   product of the two group scales (each times 64) applied by one FP32
   fused multiply-add per group, groups in ascending K; Sa * Sw in the
   epilogue.  Each group term is exact in FP32; only the cross-group FP32
   additions round. */
int mgemm_w4a4(const void *Aq, const void *As, const float *Sa, const void *Wq,
               const void *Ws, const float *Sw, void *C, int64_t M, int64_t N,
               int64_t K, int out_f32, void *stream);

/* MXFP8 grouped mixture-of-experts GLU (FlashInfer swapab_cutedsl_megakernel
   skill page, Layout section: an MXFP8 GLU MoE with an MXFP8 x MXFP8 -> BF16
   backend).  Inputs: xq [T,H] E4M3 and xs [T,H/32] E8M0 tokens; topk_ids
   [T,topk] int32 in [0,E) (entries outside that range are dropped); topk_w [T,topk] FP32 routing weights; w13q
   [E,2I,H] E4M3 with w13s [E,2I,H/32] (rows [0,I) gate, [I,2I) up); w2q
   [E,H,I] with w2s [E,H,I/32].  Per token t and slot j with expert e:
     [g;u] = x_t . w13[e]^T;  h = silu(g) * u (FP32);
     h is re-quantised to MXFP8 (E8M0 per 32 along I, OCP MX rule);
     y = h . w2[e]^T;  out[t] = sum_j topk_w[t,j] * y  (FP32), then BF16.
   out: [T,H] BF16.  ws: device workspace of at least
   mgemm_workspace_bytes(MGEMM_OP_MOE, ...) bytes (routing tables, the
   re-quantised h rows and the weighted FP32 down-projection rows, T*topk*H*4
   bytes of the total); it needs no particular contents: the call resets its
   counters on `stream` before use.  dbg_h: NULL, or a device buffer of
   T*topk*(I + I/32) bytes that receives each (token, slot) row of the
   re-quantised h (I code bytes then I/32 scale bytes) at row t*topk + j.
   H and I must be multiples of 64, topk in [1,16], E in [1,1024], T <= 2^24.
   The combine adds each token's slots in order j = 0..topk-1 in FP32 (no
   atomics): results are run-to-run bit-identical. */
int mgemm_moe_mxfp8_glu(const void *xq, const void *xs, const int32_t *topk_ids,
                        const float *topk_w, int64_t T, int64_t H, int64_t I,
                        int64_t E, int64_t topk, const void *w13q, const void *w13s,
                        const void *w2q, const void *w2s, void *out, void *ws,
                        size_t ws_bytes, void *dbg_h, void *stream);

/* mgemm_moe_mxfp8_glu with a second debug tap for stage-wise checks of the
   path: dbg_gu, NULL or a device buffer of T*topk*2*I floats (16-byte
   aligned), receives each (token, slot) row's FP32 gate/up accumulators
   g[0..I) then u[0..I) (before the GLU) at row t*topk + j; rows of dropped
   slots are not written.  Everything else as mgemm_moe_mxfp8_glu. */
int mgemm_moe_mxfp8_glu_debug(const void *xq, const void *xs, const int32_t *topk_ids,
                              const float *topk_w, int64_t T, int64_t H, int64_t I, int64_t E,
                              int64_t topk, const void *w13q, const void *w13s, const void *w2q,
                              const void *w2s, void *out, void *ws, size_t ws_bytes, void *dbg_h,
                              float *dbg_gu, void *stream);

/* The MXFP8 grouped MoE GLU above routed from the router's FP32 logits
   [T,E] in the same call: the top-k routing from the softmax of the logits
   (as mgemm_moe_route_topk computes it, bit for bit: p = softmax in FP32,
   the topk experts of largest p in descending order, equal logits to the
   lower id, weights p not renormalised) runs inside the route-prep launch
   that counts each expert's rows and ranks them, so the ids never make a
   round trip between two launches.  topk_ids [T,topk] int32 and topk_w
   [T,topk] FP32 are OUTPUTS (device buffers, 16-byte aligned) that receive
   the routing; the result equals mgemm_moe_mxfp8_glu called on them.
   logits: finite FP32, 4-byte aligned; topk <= E.  Other arguments,
   workspace, limits and errors as mgemm_moe_mxfp8_glu. */
int mgemm_moe_mxfp8_glu_logits(const void *xq, const void *xs, const float *logits, int64_t T,
                               int64_t H, int64_t I, int64_t E, int64_t topk, const void *w13q,
                               const void *w13s, const void *w2q, const void *w2s, void *out,
                               int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                               void *dbg_h, void *stream);

/* NVFP4 grouped mixture-of-experts GLU: the GLU MoE above (same FlashInfer
   skill page, which lists an NVFP4 MoE, moe_nvfp4_swapab, beside the MXFP8
   one) with every operand in NVFP4, computed on the exact FP8 route of the
   metrale_circuit hardware::exec module description (as mgemm_w4a4: NVFP4
   activations have no block-scaled MMA on gfx950).  Inputs: xq [T,H/2] E2M1
   codes (element 2j in the low nibble) and xs [T,H/16] E4M3 scales, Sx one
   FP32 tensor scale; w13q [E,2I,H/2] with w13s [E,2I,H/16] and Sw13 [E] (one
   FP32 tensor scale per expert; rows [0,I) gate, [I,2I) up); w2q [E,H,I/2]
   with w2s [E,H,I/16] and Sw2 [E]; Sh: the FP32 tensor scale under which h is
   re-quantised; topk_ids, topk_w as for the MXFP8 MoE.  Per token t, slot j,
   expert e: g, u = Sx Sw13[e] (x_t . w13[e]^T); h = silu(g) * u (FP32);
   h -> NVFP4 per 16 along I, decided in FP32: scale = E4M3(amax / 6 / Sh)
   (nearest even, saturating), code = E2M1(h / (scale * Sh)) (nearest, ties
   to the even code, saturating at 6; a zero scale gives zero codes);
   y = Sh Sw2[e] (h . w2[e]^T); out[t] = sum_j topk_w[t,j] y in FP32, BF16.
   All FP32 scales are device pointers.  ws: at least
   mgemm_workspace_bytes(MGEMM_OP_MOE_NVFP4, ...) bytes, no particular
   contents needed.  dbg_h: NULL, or T*topk*(I/2 + I/16) bytes receiving each
   (token, slot) row of the re-quantised h (I/2 code bytes, I/16 scale bytes)
   at row t*topk + j.  H a multiple of 32, I a multiple of 64, topk in
   [1,16], E in [1,1024], T <= 2^24.  Results are run-to-run bit-identical. */
int mgemm_moe_nvfp4_glu(const void *xq, const void *xs, const float *Sx,
                        const int32_t *topk_ids, const float *topk_w, int64_t T, int64_t H,
                        int64_t I, int64_t E, int64_t topk, const void *w13q,
                        const void *w13s, const float *Sw13, const void *w2q,
                        const void *w2s, const float *Sw2, const float *Sh, void *out,
                        void *ws, size_t ws_bytes, void *dbg_h, void *stream);

/* Router top-k of the MoE (top-k routing from the softmax of the router
   logits, as the mixture-of-experts GLUs above are fed; e.g. 64 experts,
   top 8).  logits: [T,E] FP32, finite.  Per token: p =
   softmax(logits) in FP32; topk_ids[t,0..topk) = the topk experts of largest
   p in descending order (chosen on the logits, which is the order of the
   exact probabilities; equal logits: the lower id first); topk_w = those p,
   not renormalised.  Outputs [T,topk] int32 / FP32, the inputs of the MoE
   entry points.  E in [1,1024], topk in [1,E], T <= 2^24; device pointers,
   4-byte aligned. */
int mgemm_moe_route_topk(const float *logits, int64_t T, int64_t E, int64_t topk,
                         int32_t *topk_ids, float *topk_w, void *stream);

/* Backward of the BF16 FFN down projection y = x . W^T (RL-Kernel PR #535's
   H3 operator; its backward names dY . W as the input gradient):
     dgrad: dX[M,K] = dY[M,N] . W[N,K]       (sum over N)
     wgrad: dW[N,K] = dY[M,N]^T . X[M,K]     (sum over M)
   BF16 operands, row-major, FP32 accumulation, BF16 output (FP32 with
   out_f32 = 1).  Each output's sum runs in one fixed order: run-to-run
   bit-identical.  ws: at least mgemm_workspace_bytes(MGEMM_OP_BF16_DGRAD /
   _WGRAD, M, N, K) bytes (the operands written contraction-major: W^T, or
   dY^T and X^T), no particular contents.  The contraction (N for dgrad, M
   for wgrad) must be a multiple of 32, K (and N for wgrad) a multiple of 8. */
int mgemm_bf16_dgrad(const void *dY, const void *W, void *dX, int64_t M, int64_t N, int64_t K,
                     int out_f32, void *ws, size_t ws_bytes, void *stream);
int mgemm_bf16_wgrad(const void *dY, const void *X, void *dW, int64_t M, int64_t N, int64_t K,
                     int out_f32, void *ws, size_t ws_bytes, void *stream);

/* workspace sizes */
enum { MGEMM_OP_BF16 = 0, MGEMM_OP_W4A16 = 1, MGEMM_OP_W4A8 = 2, MGEMM_OP_W4A4 = 3,
       MGEMM_OP_MOE = 4, MGEMM_OP_MOE_NVFP4 = 5, MGEMM_OP_BF16_DGRAD = 6,
       MGEMM_OP_BF16_WGRAD = 7 };
/* Bytes of device workspace an op needs for these sizes (0 if none).  For the
   GEMMs pass (M, N, K) and zeros; for the MoE pass (T, H, I, E, topk) in the
   T.. arguments.  Returns 0 for unknown ops or invalid sizes as well. */
size_t mgemm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t T,
                             int64_t H, int64_t I, int64_t E, int64_t topk);

/* static text for a status code */
const char *mgemm_status_string(int status);

/* library version string */
const char *mgemm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MGEMM_H */
