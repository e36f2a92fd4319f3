// kernels.h -- launcher interface between the C ABI (api.cpp) and the kernels.
// Shapes are validated by the caller; launchers only size grids and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mg {

struct W4A4Args {
  const uint8_t *aq, *as;
  const float *Sa;
  const uint8_t *wq, *ws;
  const float *Sw;
  void *C;
  int M, N, K;
  int out_f32;
};
hipError_t launch_w4a4(const W4A4Args &p, hipStream_t stream);

// BF16 activations against BF16 (w_nvfp4 = 0) or NVFP4 weights (w_nvfp4 = 1)
struct Bf16Args {
  const uint16_t *a;
  const void *w;          // uint16 [N,K] or NVFP4 codes [N,K/2]
  const uint8_t *ws;      // NVFP4 scales [N,K/16] (w_nvfp4 only)
  const float *Sw;        // NVFP4 tensor scale (w_nvfp4 only)
  void *C;
  int M, N, K;
  int out_f32;
  int w_nvfp4;
  // BF16 x BF16 tail split (set by launch_bf16): workgroups past the first
  // full_tiles each take one of `split` K ranges of a remaining tile and
  // write an FP32 partial tile to part
  int full_tiles = 0;
  int split = 1;
  float *part = nullptr;
};
// BF16 x BF16 (w_nvfp4 = 0) may split the tiles of the grid's last, partial
// round along K; the partials need bf16_workspace_bytes of ws
size_t bf16_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_bf16(const Bf16Args &p, void *ws, hipStream_t stream);
// small-M W4A16 (gemm_w4a16_dec.hip): split-K partials in the workspace
constexpr int64_t W4A16_DEC_MAX_M = 128;
size_t w4a16_dec_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_w4a16_dec(const Bf16Args &p, void *ws, hipStream_t stream);
// backward of y = x . W^T (grad_bf16.hip): operands transposed into the
// workspace, then the TN kernel
size_t bf16_grad_workspace_bytes(bool wgrad, int64_t M, int64_t N, int64_t K);  // transposes + tail partials
hipError_t launch_bf16_dgrad(const uint16_t *dY, const uint16_t *W, void *dX, int M, int N, int K,
                             int out_f32, void *ws, hipStream_t stream);
hipError_t launch_bf16_wgrad(const uint16_t *dY, const uint16_t *X, void *dW, int M, int N, int K,
                             int out_f32, void *ws, hipStream_t stream);

struct W4A8Args {
  const uint8_t *aq;
  const float *atok;
  const uint8_t *wq, *ws;
  const float *Sw;
  void *C;
  int M, N, K;
  int out_f32;
  void *work;       // split-K partials [splits, M, N] FP32
};
size_t w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int64_t w4a8_max_n();  // largest N the decode kernel's indexing supports
hipError_t launch_w4a8(const W4A8Args &p, hipStream_t stream);
// more than 32 tokens: the tiled kernel (gemm_w4a8_tile.hip) and its K split
void w4a8_tile_split(int64_t M, int64_t N, int64_t K, int &ks, int &gpw);
hipError_t launch_w4a8_tile(const W4A8Args &p, int ks, int gpw, float *part, hipStream_t stream);

struct MoeArgs {
  const uint8_t *xq, *xs;
  const int32_t *ids;
  const float *tw;
  int T, H, I, E, topk;
  const uint8_t *w13q, *w13s, *w2q, *w2s;
  uint16_t *out;
  void *ws;
  size_t ws_bytes;
  uint8_t *dbg_h;
  // non-null: route from these FP32 router logits [T,E] (softmax, top-k) in
  // the route-prep launch; ids / tw are then outputs it writes
  const float *logits;
  // optional tap: per (token, slot) row t*topk + j, the FP32 gate/up
  // accumulators g[0..I) then u[0..I)
  float *dbg_gu;
};
size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);
hipError_t launch_moe(const MoeArgs &p, hipStream_t stream);

// NVFP4 grouped MoE GLU (x, w13, w2 and h in NVFP4; tensor scales are device
// FP32: Sx, Sh one value, Sw13 / Sw2 one per expert)
struct Moe4Args {
  const uint8_t *xq, *xs;
  const float *Sx;
  const int32_t *ids;
  const float *tw;
  int T, H, I, E, topk;
  const uint8_t *w13q, *w13s;
  const float *Sw13;
  const uint8_t *w2q, *w2s;
  const float *Sw2;
  const float *Sh;
  uint16_t *out;
  void *ws;
  size_t ws_bytes;
  uint8_t *dbg_h;   // optional: per entry, I/2 code bytes then I/16 scale bytes
};
size_t moe4_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk);
// router top-k: ids / weights [T, topk] from FP32 logits [T, E] (E <= 1024)
hipError_t launch_topk_softmax(const float *logits, int T, int E, int topk, int32_t *ids,
                               float *w, hipStream_t stream);
hipError_t launch_moe4(const Moe4Args &p, hipStream_t stream);
// the grouped W4A4 GEMMs of the NVFP4 MoE (moe4.hip), on the routing that
// launch_moe4 (moe.hip) has written to the workspace
hipError_t launch_moe4_gemms(const Moe4Args &p, const int32_t *meta, const int32_t *sorted,
                             const float *wsorted, const int32_t *tile_e, const int32_t *tile_r,
                             const int32_t *tile_n, int maxtiles, uint8_t *hq, uint8_t *hs,
                             float *y, hipStream_t stream);

}  // namespace mg
