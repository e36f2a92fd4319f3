// api.cpp -- the extern "C" entry points declared in include/mgemm.h:
// execution planning, argument validation and kernel dispatch.  Every
// argument error is caught here, on the host, before anything is enqueued.
#include "../../include/mgemm.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

bool valid_fmt(int f) { return f >= MGEMM_FMT_BF16 && f <= MGEMM_FMT_MXFP8; }

bool arch_is_gfx950(const char *arch) {
  // compare the processor name, ignoring target features after ':'
  const char *name = "gfx950";
  size_t n = std::strlen(name);
  return std::strncmp(arch, name, n) == 0 && (arch[n] == '\0' || arch[n] == ':');
}

mgemm_plan_t make(int kind, int mma, int reason) {
  mgemm_plan_t p;
  p.kind = kind;
  p.mma = mma;
  p.reason = reason;
  return p;
}

// hardware::exec module docs (metrale_circuit): kind_of picks the MMA from the
// activation format; exec_of maps the pair onto the device's instructions;
// fp4_fallback sends an NVFP4 activation without an NVFP4 block-scale kernel
// to the FP8 MMA through the exact conversion; all else has no path.  gfx950's
// FP4 matrix instruction takes E8M0 scales per 32 only, so it cannot carry
// NVFP4's E4M3 scales per 16: NVFP4 activations take the exact FP8 route.
mgemm_plan_t plan_gfx950(int w, int a) {
  switch (a) {
    case MGEMM_FMT_BF16:  // BF16 MMA; the weight is widened in registers
      if (w == MGEMM_FMT_BF16 || w == MGEMM_FMT_NVFP4)
        return make(MGEMM_EXEC_NATIVE, MGEMM_MMA_BF16, MGEMM_REASON_NONE);
      return make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE, MGEMM_REASON_NO_KERNEL);
    case MGEMM_FMT_FP8_E4M3_TOKEN:  // FP8 MMA; NVFP4 weights need the exact route
      if (w == MGEMM_FMT_NVFP4)
        return make(MGEMM_EXEC_FP8_EXACT, MGEMM_MMA_FP8, MGEMM_REASON_NO_SINGLE_MMA);
      return make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE, MGEMM_REASON_NO_KERNEL);
    case MGEMM_FMT_NVFP4:  // no NVFP4 block-scale MMA here: exact FP8 route
      if (w == MGEMM_FMT_NVFP4)
        return make(MGEMM_EXEC_FP8_EXACT, MGEMM_MMA_FP8, MGEMM_REASON_NO_NVFP4_BLOCKSCALE_MMA);
      return make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE,
                  w == MGEMM_FMT_BF16 ? MGEMM_REASON_NO_INSTRUCTION : MGEMM_REASON_NO_KERNEL);
    case MGEMM_FMT_MXFP8:  // native E8M0-scaled MFMA
      if (w == MGEMM_FMT_MXFP8)
        return make(MGEMM_EXEC_NATIVE, MGEMM_MMA_MX_F8F6F4, MGEMM_REASON_NONE);
      return make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE, MGEMM_REASON_NO_KERNEL);
  }
  return make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE, MGEMM_REASON_NO_KERNEL);
}

// per-device architecture cache (the only state the library keeps)
constexpr int kMaxDev = 64;
std::once_flag g_arch_once[kMaxDev];
char g_arch[kMaxDev][64];
hipError_t g_arch_err[kMaxDev];

hipError_t device_arch(int dev, const char **arch) {
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::call_once(g_arch_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_arch_err[dev] = hipGetDeviceProperties(&prop, dev);
    if (g_arch_err[dev] == hipSuccess) {
      std::strncpy(g_arch[dev], prop.gcnArchName, sizeof(g_arch[dev]) - 1);
      g_arch[dev][sizeof(g_arch[dev]) - 1] = '\0';
    }
  });
  *arch = g_arch[dev];
  return g_arch_err[dev];
}

bool debug_on() {
  static int on = [] {
    const char *e = std::getenv("MGEMM_DEBUG");
    return (e && e[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxDim = 0x7FFFFFFF;

int check_mnk(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return MGEMM_ERR_SHAPE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return MGEMM_ERR_SHAPE;
  // every byte offset the kernels form must fit in int64 comfortably
  if ((double)M * (double)K > 4.0e18 || (double)N * (double)K > 4.0e18 ||
      (double)M * (double)N * 4.0 > 4.0e18)
    return MGEMM_ERR_SHAPE;
  return MGEMM_OK;
}

// the pair must have a path on the calling thread's current device
int check_path(int w, int a) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MGEMM_ERR_HIP;
  const char *arch = nullptr;
  if (device_arch(dev, &arch) != hipSuccess) return MGEMM_ERR_HIP;
  mgemm_plan_t p = arch_is_gfx950(arch) ? plan_gfx950(w, a)
                                        : make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE,
                                               MGEMM_REASON_UNSUPPORTED_DEVICE);
  return p.kind == MGEMM_EXEC_NOPATH ? MGEMM_ERR_NOPATH : MGEMM_OK;
}

int finish(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    if (debug_on()) std::fprintf(stderr, "mgemm: %s: %s\n", what, hipGetErrorString(e));
    return MGEMM_ERR_HIP;
  }
  return MGEMM_OK;
}

// the MXFP8 MoE entry points: routing ids / weights given (logits == NULL),
// or routed from FP32 router logits, ids / weights then written by the call
int moe_mxfp8(const void *xq, const void *xs, const float *logits, const int32_t *topk_ids,
              const float *topk_w, int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk,
              const void *w13q, const void *w13s, const void *w2q, const void *w2s, void *out,
              void *ws, size_t ws_bytes, void *dbg_h, float *dbg_gu, void *stream,
              const char *what) {
  if (!xq || !xs || !topk_ids || !topk_w || !w13q || !w13s || !w2q || !w2s || !out)
    return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(topk_ids) || !aligned16(topk_w) ||
      !aligned16(w13q) || !aligned16(w13s) || !aligned16(w2q) || !aligned16(w2s) ||
      !aligned16(out) || (dbg_h && !aligned16(dbg_h)) || (dbg_gu && !aligned16(dbg_gu)))
    return MGEMM_ERR_INVALID_ARG;
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return MGEMM_ERR_SHAPE;
  if (H % 64 != 0 || I % 64 != 0 || topk > 16 || E > 1024 || T > (1 << 24) ||
      H > (1 << 20) || I > (1 << 20) || (double)T * topk * (double)(H > I ? H : I) > 4.0e18)
    return MGEMM_ERR_SHAPE;
  if (int rc = check_path(MGEMM_FMT_MXFP8, MGEMM_FMT_MXFP8)) return rc;
  const size_t need = mg::moe_workspace_bytes(T, H, I, E, topk);
  if (!ws || ws_bytes < need || !aligned16(ws)) return MGEMM_ERR_WORKSPACE;
  mg::MoeArgs p{(const uint8_t *)xq, (const uint8_t *)xs, topk_ids, topk_w, (int)T, (int)H,
                (int)I, (int)E, (int)topk, (const uint8_t *)w13q, (const uint8_t *)w13s,
                (const uint8_t *)w2q, (const uint8_t *)w2s, (uint16_t *)out, ws, ws_bytes,
                (uint8_t *)dbg_h, logits, dbg_gu};
  return finish(mg::launch_moe(p, (hipStream_t)stream), what);
}

}  // namespace

extern "C" {

int mgemm_plan_arch(const char *gcn_arch, int w_fmt, int a_fmt, mgemm_plan_t *out) {
  if (!gcn_arch || !out || !valid_fmt(w_fmt) || !valid_fmt(a_fmt)) return MGEMM_ERR_INVALID_ARG;
  *out = arch_is_gfx950(gcn_arch)
             ? plan_gfx950(w_fmt, a_fmt)
             : make(MGEMM_EXEC_NOPATH, MGEMM_MMA_NONE, MGEMM_REASON_UNSUPPORTED_DEVICE);
  return MGEMM_OK;
}

int mgemm_plan(int device, int w_fmt, int a_fmt, mgemm_plan_t *out) {
  if (!out || !valid_fmt(w_fmt) || !valid_fmt(a_fmt)) return MGEMM_ERR_INVALID_ARG;
  const char *arch = nullptr;
  if (device_arch(device, &arch) != hipSuccess) return MGEMM_ERR_HIP;
  return mgemm_plan_arch(arch, w_fmt, a_fmt, out);
}

int mgemm_pair_name(int w_fmt, int a_fmt, char *buf, size_t len) {
  if (!valid_fmt(w_fmt) || !valid_fmt(a_fmt) || !buf || len == 0) return MGEMM_ERR_INVALID_ARG;
  static const int bits[4] = {16, 4, 8, 8};
  int n = std::snprintf(buf, len, "W%dA%d", bits[w_fmt], bits[a_fmt]);
  if (n < 0 || (size_t)n >= len) return MGEMM_ERR_INVALID_ARG;
  return n;
}

int mgemm_bf16(const void *A, const void *W, void *C, int64_t M, int64_t N, int64_t K,
               int out_f32, void *ws, size_t ws_bytes, void *stream) {
  if (!A || !W || !C || (out_f32 != 0 && out_f32 != 1)) return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(W) || !aligned16(C)) return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(M, N, K)) return rc;
  if (int rc = check_path(MGEMM_FMT_BF16, MGEMM_FMT_BF16)) return rc;
  const size_t need = mg::bf16_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MGEMM_ERR_WORKSPACE;
  mg::Bf16Args p{(const uint16_t *)A, W, nullptr, nullptr, C, (int)M, (int)N, (int)K, out_f32, 0};
  return finish(mg::launch_bf16(p, need > 0 ? ws : nullptr, (hipStream_t)stream), "mgemm_bf16");
}

int mgemm_w4a16(const void *A, const void *Wq, const void *Ws, const float *Sw, void *C,
                int64_t M, int64_t N, int64_t K, int out_f32, void *ws, size_t ws_bytes,
                void *stream) {
  if (!A || !Wq || !Ws || !Sw || !C || (out_f32 != 0 && out_f32 != 1)) return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(Wq) || !aligned16(Ws) || !aligned16(Sw) || !aligned16(C))
    return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(M, N, K)) return rc;
  const size_t need = mg::w4a16_dec_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MGEMM_ERR_WORKSPACE;
  if (int rc = check_path(MGEMM_FMT_NVFP4, MGEMM_FMT_BF16)) return rc;
  mg::Bf16Args p{(const uint16_t *)A, Wq, (const uint8_t *)Ws, Sw, C, (int)M, (int)N, (int)K,
                 out_f32, 1};
  if (need > 0) return finish(mg::launch_w4a16_dec(p, ws, (hipStream_t)stream), "mgemm_w4a16");
  return finish(mg::launch_bf16(p, nullptr, (hipStream_t)stream), "mgemm_w4a16");
}

int mgemm_w4a8(const void *Aq, const float *a_tok, const void *Wq, const void *Ws,
               const float *Sw, void *C, int64_t M, int64_t N, int64_t K, int out_f32,
               void *ws, size_t ws_bytes, void *stream) {
  if (!Aq || !a_tok || !Wq || !Ws || !Sw || !C || (out_f32 != 0 && out_f32 != 1))
    return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(Aq) || !aligned16(a_tok) || !aligned16(Wq) || !aligned16(Ws) ||
      !aligned16(Sw) || !aligned16(C))
    return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(M, N, K)) return rc;
  if (N > mg::w4a8_max_n()) return MGEMM_ERR_SHAPE;
  const size_t need = mg::w4a8_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return MGEMM_ERR_WORKSPACE;
  if (int rc = check_path(MGEMM_FMT_NVFP4, MGEMM_FMT_FP8_E4M3_TOKEN)) return rc;
  mg::W4A8Args p{(const uint8_t *)Aq, a_tok, (const uint8_t *)Wq, (const uint8_t *)Ws, Sw, C,
                 (int)M, (int)N, (int)K, out_f32, need > 0 ? ws : nullptr};
  return finish(mg::launch_w4a8(p, (hipStream_t)stream), "mgemm_w4a8");
}

int mgemm_w4a4(const void *Aq, const void *As, const float *Sa, const void *Wq, const void *Ws,
               const float *Sw, void *C, int64_t M, int64_t N, int64_t K, int out_f32,
               void *stream) {
  if (!Aq || !As || !Sa || !Wq || !Ws || !Sw || !C || (out_f32 != 0 && out_f32 != 1))
    return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(Aq) || !aligned16(As) || !aligned16(Sa) || !aligned16(Wq) || !aligned16(Ws) ||
      !aligned16(Sw) || !aligned16(C))
    return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(M, N, K)) return rc;
  if (int rc = check_path(MGEMM_FMT_NVFP4, MGEMM_FMT_NVFP4)) return rc;
  mg::W4A4Args p{(const uint8_t *)Aq, (const uint8_t *)As, Sa, (const uint8_t *)Wq,
                 (const uint8_t *)Ws, Sw, C, (int)M, (int)N, (int)K, out_f32};
  return finish(mg::launch_w4a4(p, (hipStream_t)stream), "mgemm_w4a4");
}

int mgemm_moe_mxfp8_glu(const void *xq, const void *xs, const int32_t *topk_ids,
                        const float *topk_w, int64_t T, int64_t H, int64_t I, int64_t E,
                        int64_t topk, const void *w13q, const void *w13s, const void *w2q,
                        const void *w2s, void *out, void *ws, size_t ws_bytes, void *dbg_h,
                        void *stream) {
  return moe_mxfp8(xq, xs, nullptr, topk_ids, topk_w, T, H, I, E, topk, w13q, w13s, w2q, w2s, out,
                   ws, ws_bytes, dbg_h, nullptr, stream, "mgemm_moe_mxfp8_glu");
}

int mgemm_moe_mxfp8_glu_debug(const void *xq, const void *xs, const int32_t *topk_ids,
                              const float *topk_w, int64_t T, int64_t H, int64_t I, int64_t E,
                              int64_t topk, const void *w13q, const void *w13s, const void *w2q,
                              const void *w2s, void *out, void *ws, size_t ws_bytes, void *dbg_h,
                              float *dbg_gu, void *stream) {
  return moe_mxfp8(xq, xs, nullptr, topk_ids, topk_w, T, H, I, E, topk, w13q, w13s, w2q, w2s, out,
                   ws, ws_bytes, dbg_h, dbg_gu, stream, "mgemm_moe_mxfp8_glu_debug");
}

int mgemm_moe_mxfp8_glu_logits(const void *xq, const void *xs, const float *logits, int64_t T,
                               int64_t H, int64_t I, int64_t E, int64_t topk, const void *w13q,
                               const void *w13s, const void *w2q, const void *w2s, void *out,
                               int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                               void *dbg_h, void *stream) {
  if (!logits) return MGEMM_ERR_INVALID_ARG;
  if ((uintptr_t)logits & 3) return MGEMM_ERR_INVALID_ARG;
  if (topk > E) return MGEMM_ERR_SHAPE;
  return moe_mxfp8(xq, xs, logits, topk_ids, topk_w, T, H, I, E, topk, w13q, w13s, w2q, w2s, out,
                   ws, ws_bytes, dbg_h, nullptr, stream, "mgemm_moe_mxfp8_glu_logits");
}

int mgemm_moe_nvfp4_glu(const void *xq, const void *xs, const float *Sx,
                        const int32_t *topk_ids, const float *topk_w, int64_t T, int64_t H,
                        int64_t I, int64_t E, int64_t topk, const void *w13q,
                        const void *w13s, const float *Sw13, const void *w2q,
                        const void *w2s, const float *Sw2, const float *Sh, void *out,
                        void *ws, size_t ws_bytes, void *dbg_h, void *stream) {
  if (!xq || !xs || !Sx || !topk_ids || !topk_w || !w13q || !w13s || !Sw13 || !w2q || !w2s ||
      !Sw2 || !Sh || !out)
    return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(topk_ids) || !aligned16(topk_w) ||
      !aligned16(w13q) || !aligned16(w13s) || !aligned16(w2q) || !aligned16(w2s) ||
      !aligned16(out) || ((uintptr_t)Sx & 3) || ((uintptr_t)Sw13 & 3) || ((uintptr_t)Sw2 & 3) ||
      ((uintptr_t)Sh & 3))
    return MGEMM_ERR_INVALID_ARG;
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return MGEMM_ERR_SHAPE;
  if (H % 32 != 0 || I % 64 != 0 || topk > 16 || E > 1024 || T > (1 << 24) ||
      H > (1 << 20) || I > (1 << 20) || (double)T * topk * (double)(H > I ? H : I) > 4.0e18)
    return MGEMM_ERR_SHAPE;
  if (int rc = check_path(MGEMM_FMT_NVFP4, MGEMM_FMT_NVFP4)) return rc;
  const size_t need = mg::moe4_workspace_bytes(T, H, I, E, topk);
  if (!ws || ws_bytes < need || !aligned16(ws)) return MGEMM_ERR_WORKSPACE;
  mg::Moe4Args p{(const uint8_t *)xq, (const uint8_t *)xs, Sx, topk_ids, topk_w, (int)T, (int)H,
                 (int)I, (int)E, (int)topk, (const uint8_t *)w13q, (const uint8_t *)w13s, Sw13,
                 (const uint8_t *)w2q, (const uint8_t *)w2s, Sw2, Sh, (uint16_t *)out, ws,
                 ws_bytes, (uint8_t *)dbg_h};
  return finish(mg::launch_moe4(p, (hipStream_t)stream), "mgemm_moe_nvfp4_glu");
}

int mgemm_bf16_dgrad(const void *dY, const void *W, void *dX, int64_t M, int64_t N, int64_t K,
                     int out_f32, void *ws, size_t ws_bytes, void *stream) {
  if (!dY || !W || !dX || (out_f32 != 0 && out_f32 != 1)) return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(dY) || !aligned16(W) || !aligned16(dX)) return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(M, K, N)) return rc;            // contraction over N
  if (K % 8 != 0) return MGEMM_ERR_SHAPE;
  if (int rc = check_path(MGEMM_FMT_BF16, MGEMM_FMT_BF16)) return rc;
  if (!ws || !aligned16(ws) || ws_bytes < mg::bf16_grad_workspace_bytes(false, M, N, K))
    return MGEMM_ERR_WORKSPACE;
  return finish(mg::launch_bf16_dgrad((const uint16_t *)dY, (const uint16_t *)W, dX, (int)M,
                                      (int)N, (int)K, out_f32, ws, (hipStream_t)stream),
                "mgemm_bf16_dgrad");
}

int mgemm_bf16_wgrad(const void *dY, const void *X, void *dW, int64_t M, int64_t N, int64_t K,
                     int out_f32, void *ws, size_t ws_bytes, void *stream) {
  if (!dY || !X || !dW || (out_f32 != 0 && out_f32 != 1)) return MGEMM_ERR_INVALID_ARG;
  if (!aligned16(dY) || !aligned16(X) || !aligned16(dW)) return MGEMM_ERR_INVALID_ARG;
  if (int rc = check_mnk(N, K, M)) return rc;            // contraction over M
  if (N % 8 != 0 || K % 8 != 0) return MGEMM_ERR_SHAPE;
  if (int rc = check_path(MGEMM_FMT_BF16, MGEMM_FMT_BF16)) return rc;
  if (!ws || !aligned16(ws) || ws_bytes < mg::bf16_grad_workspace_bytes(true, M, N, K))
    return MGEMM_ERR_WORKSPACE;
  return finish(mg::launch_bf16_wgrad((const uint16_t *)dY, (const uint16_t *)X, dW, (int)M,
                                      (int)N, (int)K, out_f32, ws, (hipStream_t)stream),
                "mgemm_bf16_wgrad");
}

int mgemm_moe_route_topk(const float *logits, int64_t T, int64_t E, int64_t topk,
                         int32_t *topk_ids, float *topk_w, void *stream) {
  if (!logits || !topk_ids || !topk_w) return MGEMM_ERR_INVALID_ARG;
  if (((uintptr_t)logits & 3) || ((uintptr_t)topk_ids & 3) || ((uintptr_t)topk_w & 3))
    return MGEMM_ERR_INVALID_ARG;
  if (T <= 0 || E <= 0 || topk <= 0 || topk > E || E > 1024 || T > (1 << 24))
    return MGEMM_ERR_SHAPE;
  return finish(mg::launch_topk_softmax(logits, (int)T, (int)E, (int)topk, topk_ids, topk_w,
                                        (hipStream_t)stream),
                "mgemm_moe_route_topk");
}

size_t mgemm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t T, int64_t H,
                             int64_t I, int64_t E, int64_t topk) {
  switch (op) {
    case MGEMM_OP_W4A4:
      return 0;
    case MGEMM_OP_BF16:
      if (check_mnk(M, N, K) != MGEMM_OK) return 0;
      return mg::bf16_workspace_bytes(M, N, K);
    case MGEMM_OP_W4A16:
      if (check_mnk(M, N, K) != MGEMM_OK) return 0;
      return mg::w4a16_dec_workspace_bytes(M, N, K);
    case MGEMM_OP_W4A8:
      if (check_mnk(M, N, K) != MGEMM_OK) return 0;
      return mg::w4a8_workspace_bytes(M, N, K);
    case MGEMM_OP_MOE:
      if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0 || topk > 16 || E > 1024 ||
          H % 64 != 0 || I % 64 != 0)
        return 0;
      return mg::moe_workspace_bytes(T, H, I, E, topk);
    case MGEMM_OP_BF16_DGRAD:
      if (check_mnk(M, K, N) != MGEMM_OK || K % 8 != 0) return 0;
      return mg::bf16_grad_workspace_bytes(false, M, N, K);
    case MGEMM_OP_BF16_WGRAD:
      if (check_mnk(N, K, M) != MGEMM_OK || N % 8 != 0 || K % 8 != 0) return 0;
      return mg::bf16_grad_workspace_bytes(true, M, N, K);
    case MGEMM_OP_MOE_NVFP4:
      if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0 || topk > 16 || E > 1024 ||
          H % 32 != 0 || I % 64 != 0)
        return 0;
      return mg::moe4_workspace_bytes(T, H, I, E, topk);
  }
  return 0;
}

const char *mgemm_status_string(int status) {
  switch (status) {
    case MGEMM_OK: return "ok";
    case MGEMM_ERR_INVALID_ARG: return "invalid argument (NULL, misaligned pointer or bad enum)";
    case MGEMM_ERR_SHAPE: return "invalid shape";
    case MGEMM_ERR_NOPATH: return "no execution path for this format pair on this device";
    case MGEMM_ERR_WORKSPACE: return "workspace missing or too small";
    case MGEMM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *mgemm_version(void) { return "mgemm 0.1 (gfx950)"; }

}  // extern "C"
