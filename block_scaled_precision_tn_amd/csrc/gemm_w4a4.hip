// gemm_w4a4.hip -- NVFP4 x NVFP4 TN GEMM on gfx950 through the exact E4M3
// route of the metrale_circuit hardware::exec module description:
//
//   * both operands' E2M1 codes become E4M3 bytes by the mask-and-shift bit
//     identity (value x 2^-6), giving FP8 MFMA operands;
//   * one v_mfma_f32_32x32x16_fp8_fp8 per 16-element group with a zero
//     accumulator gives the group partial P_g (exact in FP32);
//   * the two group scales, each decoded and multiplied by 64 (the folded
//     2^6), form c_g = (64 s_a)(64 s_w) -- exact, computed here as a 32x32
//     outer product on the BF16 MFMA (one non-zero K slot), which keeps the
//     per-element scale products off the vector ALU;
//   * acc = fma(c_g, P_g, acc) in FP32, groups in ascending K;
//   * epilogue: acc * (S_a * S_w), BF16 (nearest even) or FP32 store.
//
// Workgroup: 256 threads (4 waves, 2x2), tile 128 x 128, wave tile 64 x 64
// (2 x 2 MFMA blocks of 32 x 32).  K is staged through LDS 128 elements (8
// groups) at a time, double-buffered, fed by 16-byte global loads.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int GPS = 8;              // groups (of 16 K-elements) per LDS stage
constexpr int CODE_ROW = 64 + 16;   // LDS bytes per tile row of codes (32 B per half + pad)
constexpr int SC_ROW = 16;          // LDS bytes per tile row of scales (8 x bf16)

struct StageRegs {
  u32x4 code[2][2];   // [operand][chunk]
  u32x2 sc;           // raw scale bytes of one row (threads < 128: A, else W)
};

__device__ __forceinline__ void load_stage(const W4A4Args &p, int m0, int n0, int g0, int G,
                                           int tid, StageRegs &r) {
  const int64_t rowb = p.K / 2, rows = p.K / 16;
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    const uint8_t *base = op == 0 ? p.aq : p.wq;
    const int R = op == 0 ? p.M : p.N, o = op == 0 ? m0 : n0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 2, c16 = c & 3;
      const int g = g0 + 2 * c16;
      int grow = o + row;
      grow = grow < R ? grow : R - 1;
      const int gs = g < G ? g : G - 2;   // in-bounds address; data masked below
      const u32x4 v = *(const u32x4 *)(base + (int64_t)grow * rowb + (int64_t)gs * 8);
      r.code[op][i] = g < G ? v : u32x4{0, 0, 0, 0};
    }
  }
  {
    const int op = tid >> 7, row = tid & 127;
    const uint8_t *base = op == 0 ? p.as : p.ws;
    const int R = op == 0 ? p.M : p.N, o = op == 0 ? m0 : n0;
    int grow = o + row;
    grow = grow < R ? grow : R - 1;
    const uint16_t *s16 = (const uint16_t *)(base + (int64_t)grow * rows);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int g = g0 + 2 * q;
      const uint32_t v = s16[(g < G ? g : G - 2) >> 1];
      w[q] = g < G ? v : 0u;
    }
    r.sc = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
  }
}

__device__ __forceinline__ void store_stage(uint8_t *lds_code, uint8_t *lds_sc, int tid,
                                            const StageRegs &r) {
#pragma unroll
  for (int op = 0; op < 2; ++op) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 2, c16 = c & 3;
      uint8_t *dst = lds_code + op * (BM * CODE_ROW) + row * CODE_ROW;
      // global chunk = (g,h0) (g,h1) (g+1,h0) (g+1,h1); LDS row = [h0: g0..g7][h1: g0..g7]
      *(u32x2 *)(dst + 8 * c16) = u32x2{r.code[op][i][0], r.code[op][i][2]};
      *(u32x2 *)(dst + 32 + 8 * c16) = u32x2{r.code[op][i][1], r.code[op][i][3]};
    }
  }
  {
    const int op = tid >> 7, row = tid & 127;
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = q < 2 ? r.sc[0] : r.sc[1];
      const uint32_t b0 = (w >> (16 * (q & 1))) & 0xFF, b1 = (w >> (16 * (q & 1) + 8)) & 0xFF;
      v[q] = e4m3_x64_to_bf16(b0) | (e4m3_x64_to_bf16(b1) << 16);
    }
    *(u32x4 *)(lds_sc + op * (BM * SC_ROW) + row * SC_ROW) = v;
  }
}

__global__ __launch_bounds__(256, 2) void w4a4_fp8route_kernel(W4A4Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_code[2][2 * BM * CODE_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t lds_sc[2][2 * BM * SC_ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = p.K / 16;
  const int S = (G + GPS - 1) / GPS;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};
  const f32x16 zero = {0};

  StageRegs st;
  load_stage(p, m0, n0, 0, G, tid, st);
  store_stage(lds_code[0], lds_sc[0], tid, st);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const int buf = s & 1;
    if (s + 1 < S) load_stage(p, m0, n0, (s + 1) * GPS, G, tid, st);

    const uint8_t *ca = lds_code[buf] + (wm * 64 + l32) * CODE_ROW + 32 * h;
    const uint8_t *cw = lds_code[buf] + BM * CODE_ROW + (wn * 64 + l32) * CODE_ROW + 32 * h;
    const uint8_t *sca = lds_sc[buf] + (wm * 64 + l32) * SC_ROW;
    const uint8_t *scw = lds_sc[buf] + BM * SC_ROW + (wn * 64 + l32) * SC_ROW;
#pragma unroll 1
    for (int g = 0; g < GPS; ++g) {
      uint64_t fa[2], fw[2];
      u32x4 sa[2], sw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = nvfp4x8_to_e4m3x8(*(const uint32_t *)(ca + i * 32 * CODE_ROW + 4 * g));
        fw[i] = nvfp4x8_to_e4m3x8(*(const uint32_t *)(cw + i * 32 * CODE_ROW + 4 * g));
        // outer-product operands: K slot 0 carries the scale (lanes 0..31), all else 0
        const uint32_t a16 = *(const uint16_t *)(sca + i * 32 * SC_ROW + 2 * g);
        const uint32_t w16 = *(const uint16_t *)(scw + i * 32 * SC_ROW + 2 * g);
        sa[i] = u32x4{h == 0 ? a16 : 0u, 0u, 0u, 0u};
        sw[i] = u32x4{h == 0 ? w16 : 0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x16 pg = mfma_fp8(fa[i], fw[j], zero);
          const f32x16 cg = mfma_bf16(sa[i], sw[j], zero);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(cg[r], pg[r], acc[i][j][r]);
        }
    }

    if (s + 1 < S) store_stage(lds_code[buf ^ 1], lds_sc[buf ^ 1], tid, st);
    __syncthreads();
  }

  const float gs = *p.Sa * *p.Sw;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + l32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
        const float v = acc[i][j][r] * gs;
        if (p.out_f32)
          ((float *)p.C)[(int64_t)row * p.N + col] = v;
        else
          ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

}  // namespace

hipError_t launch_w4a4(const W4A4Args &p, hipStream_t stream) {
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM);
  hipLaunchKernelGGL(w4a4_fp8route_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mg
