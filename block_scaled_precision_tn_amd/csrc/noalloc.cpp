// noalloc.cpp -- W4A8 entry point that allocates nothing, for callers that
// cannot call hipMalloc (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// mgemm_w4a8 takes its split-K partials in a caller-provided workspace; this
// variant takes them from `scratch`, a file-scope device array of fixed size
// that every GPU the library runs on holds until the process ends.  In host
// code the array's name is only a host-side stand-in: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and that address, never the name, is what the kernels receive.
#include "../../include/mgemm.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = MGEMM_W4A8_NOALLOC_MAX_WS;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDev = 64;
std::once_flag g_once[kMaxDev];
void *g_ptr[kMaxDev];
hipError_t g_err[kMaxDev];

// the device address of this device's copy of `scratch` (set up on the first
// call on each device, with that device current)
hipError_t scratch_ptr(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace

extern "C" int mgemm_w4a8_noalloc(const void *Aq, const float *a_tok, const void *Wq,
                                  const void *Ws, const float *Sw, void *C, int64_t M, int64_t N,
                                  int64_t K, int out_f32, void *stream) {
  // argument and shape checks first: the same rules as mgemm_w4a8, which
  // sizes nothing here (a workspace of 0 bytes passes only when none is needed)
  if (!Aq || !a_tok || !Wq || !Ws || !Sw || !C) return MGEMM_ERR_INVALID_ARG;
  const size_t need = mgemm_workspace_bytes(MGEMM_OP_W4A8, M, N, K, 0, 0, 0, 0, 0);
  if (need > kScratchBytes) return MGEMM_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MGEMM_ERR_HIP;
  void *ws = nullptr;
  if (scratch_ptr(dev, &ws) != hipSuccess || !ws) return MGEMM_ERR_HIP;
  return mgemm_w4a8(Aq, a_tok, Wq, Ws, Sw, C, M, N, K, out_f32, ws, kScratchBytes, stream);
}
