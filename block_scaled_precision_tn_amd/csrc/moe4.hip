// moe4.hip -- the grouped GEMMs of the NVFP4 GLU mixture of experts on
// gfx950.  The MoE is the GLU MoE of the FlashInfer swapab_cutedsl_megakernel
// skill page (Layout section; the page lists an NVFP4 MoE, moe_nvfp4_swapab,
// beside the MXFP8 one) with every operand in NVFP4: E2M1 codes, an E4M3
// scale per 16 K-elements and an FP32 tensor scale (one per expert for the
// weights).  NVFP4 activations have no block-scaled MMA on gfx950, so both
// GEMMs take the exact FP8 route of the metrale_circuit hardware::exec module
// description, as the W4A4 GEMM does: codes -> E4M3 by the bit identity
// (value x 2^-6), one v_mfma_f32_32x32x16_fp8_fp8 per 16-element group with a
// zero accumulator, the group's scale product s_a * s_w formed on the matrix
// unit from the raw scale bytes, acc = fma(s_a s_w, P'_g, acc) in FP32 in
// ascending K, the folded 2^12 and the tensor scales in the epilogue.
//
//   k4_gemm<true>  gate/up over expert-sorted routed rows (token rows
//                  gathered): B rows [0,64) = gate rows c0.., [64,128) = up
//                  rows I+c0.., so each wave's two 32x32 blocks hold g and u
//                  of the same columns; epilogue h = silu(g) * u and NVFP4
//                  re-quantisation under the tensor scale Sh (per 16 columns:
//                  scale = E4M3(amax / 6 / Sh), code = E2M1(h / (scale Sh)),
//                  taken in FP32), h stored in sorted order
//   k4_gemm<false> down: sorted h rows against w2[e]; epilogue times the
//                  routing weight, FP32 rows for the ordered combine
// Workgroup: 512 threads (8 waves, 4x2), tile 128 routed rows x 128 weight
// rows, wave tile 32 x 64, K staged 64 at a time (4 groups) through two LDS
// buffers with global loads two stages ahead (the W4A4 kernel's layout: each
// (32-row block, group) operand contiguous in lane order).
#include "common.h"
#include "kernels.h"
#include "quant.h"

namespace mg {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int GPS = 4;        // groups (of 16 K-elements) per LDS stage

__device__ __forceinline__ int coff(int row, int g, int h) {
  return ((((row >> 5) * GPS + g) * 64) + h * 32 + (row & 31)) * 8;
}

struct Stage {
  uint8_t code[2][BM * GPS * 16];
  uint64_t sc[2][GPS * BM];   // [group][row]: raw E4M3 scale byte, zero-extended to 8 bytes
};

struct StageRegs {
  u32x4 code;      // 32 codes (groups 2q, 2q+1) of one row
  uint32_t s0, s1; // scale bytes of groups (0, 1) and (2, 3) of one row
};

// the rows this thread loads: codes of row (tid & 255) / 2 (A for threads
// < 256, else B), scales of row tid & 127 (A for (tid / 128) even, else B)
struct Rows {
  const uint8_t *code;
  const uint16_t *sc;
};

__device__ __forceinline__ void load_stage(const Rows &rw, int g0, int G, int tid, StageRegs &r) {
  const int g = g0 + 2 * (tid & 1);       // G is even (K % 32 == 0): g < G covers g + 1
  r.code = *(const u32x4 *)(rw.code + (int64_t)(g < G ? g : G - 2) * 8);
  r.s0 = rw.sc[(g0 < G ? g0 : G - 2) >> 1];
  r.s1 = rw.sc[(g0 + 2 < G ? g0 + 2 : G - 2) >> 1];
}

__device__ __forceinline__ void store_stage(Stage &s, int tid, const StageRegs &r, int g0, int G) {
  {
    const int row = (tid & 255) >> 1, q = tid & 1;
    const int op = tid >> 8;
    const u32x4 v = g0 + 2 * q < G ? r.code : u32x4{0, 0, 0, 0};
    const uint64_t e0 = nvfp4x8_to_e4m3x8(v[0]), e1 = nvfp4x8_to_e4m3x8(v[1]);
    const uint64_t e2 = nvfp4x8_to_e4m3x8(v[2]), e3 = nvfp4x8_to_e4m3x8(v[3]);
    uint8_t *c = s.code[op];
    *(uint64_t *)(c + coff(row, 2 * q, 0)) = e0;
    *(uint64_t *)(c + coff(row, 2 * q, 1)) = e1;
    *(uint64_t *)(c + coff(row, 2 * q + 1, 0)) = e2;
    *(uint64_t *)(c + coff(row, 2 * q + 1, 1)) = e3;
  }
  if (tid < 256) {
    const uint32_t w = (g0 < G ? r.s0 : 0u) | ((g0 + 2 < G ? r.s1 : 0u) << 16);
#pragma unroll
    for (int g = 0; g < GPS; ++g) s.sc[tid >> 7][g * BM + (tid & 127)] = (w >> (8 * g)) & 0xFFu;
  }
}

template <bool GU>
__global__ __launch_bounds__(512, 2) void k4_gemm(Moe4Args p, const int32_t *meta,
                                                  const int32_t *sorted, const float *wsorted,
                                                  const int32_t *tile_e, const int32_t *tile_r,
                                                  const int32_t *tile_n, uint8_t *hq, uint8_t *hs,
                                                  float *y) {
  __shared__ __attribute__((aligned(16))) Stage lds[2];
  __shared__ uint64_t zsc[GPS * BM];   // zeros: the A-side scale operand of lanes h = 1
  __shared__ float s_w[BM];            // routing weight of each tile row (down)
  const int tile = blockIdx.y;
  if (tile >= meta[0]) return;
  const int e = tile_e[tile], r0 = tile_r[tile], nrows = tile_n[tile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, h = lane >> 5;
  const int H = p.H, I = p.I, K = GU ? H : I, G = K / 16, S = (G + GPS - 1) / GPS;
  const int c0 = blockIdx.x * (GU ? 64 : BN);

  // A row r: the token (gate/up) or the sorted h row (down) of routed row
  // r0 + r; rows past the tile repeat its first row (never stored).  B row q:
  // gate / up row of w13[e], or row of w2[e] (past H: the last, never stored).
  auto arow = [&](int r) -> int64_t {
    const int rr = r0 + (r < nrows ? r : 0);
    return GU ? (int64_t)(sorted[rr] / p.topk) : (int64_t)rr;
  };
  auto brow = [&](int q) -> int64_t {
    if (GU) return (int64_t)e * 2 * I + (q < 64 ? c0 + q : I + c0 + q - 64);
    return (int64_t)e * H + (c0 + q < H ? c0 + q : H - 1);
  };
  const uint8_t *aq = GU ? p.xq : hq, *as = GU ? p.xs : hs;
  const uint8_t *bq = GU ? p.w13q : p.w2q, *bs = GU ? p.w13s : p.w2s;
  Rows rw;
  {
    const int row = (tid & 255) >> 1, srow = tid & 127;
    rw.code = tid < 256 ? aq + arow(row) * (K / 2) : bq + brow(row) * (K / 2);
    rw.sc = (const uint16_t *)(((tid >> 7) & 1) ? bs + brow(srow) * G : as + arow(srow) * G);
  }
  // (down) the tile rows' routing weights, requested before the main loop
  const float wv = GU ? 0.0f : wsorted[r0 + ((tid & 127) < nrows ? (tid & 127) : 0)];

  // the wave's two 32-row B blocks: gate and up of the same columns, or two
  // adjacent blocks of w2 rows
  const int ob0 = GU ? wn * 32 : wn * 64, ob1 = GU ? 64 + wn * 32 : wn * 64 + 32;
  f32x16 acc[2] = {f32x16{0}, f32x16{0}};
  const f32x16 zero = {0};
  auto compute = [&](const Stage &cur) {
    const uint8_t *pa = cur.code[0] + coff(wm * 32, 0, 0) + 8 * lane;
    const uint8_t *pw0 = cur.code[1] + coff(ob0, 0, 0) + 8 * lane;
    const uint8_t *pw1 = cur.code[1] + coff(ob1, 0, 0) + 8 * lane;
    // scale operands: lane (row, h = 0) holds its row's scale byte at K = 0
    // and zeros elsewhere; on the A side lanes h = 1 read zeros, so the K = 16
    // product is exactly s_a * s_w
    const uint64_t *psa = (h ? zsc : cur.sc[0]) + wm * 32 + l32;
    const uint64_t *psw0 = cur.sc[1] + ob0 + l32, *psw1 = cur.sc[1] + ob1 + l32;
#pragma unroll 1
    for (int g = 0; g < GPS; ++g) {
      const uint64_t a = *(const uint64_t *)(pa + 512 * g);
      const uint64_t w0 = *(const uint64_t *)(pw0 + 512 * g), w1 = *(const uint64_t *)(pw1 + 512 * g);
      const uint64_t sa = psa[BM * g], sw0 = psw0[BM * g], sw1 = psw1[BM * g];
      const f32x16 c0v = mfma_fp8(sa, sw0, zero);
      const f32x16 c1v = mfma_fp8(sa, sw1, zero);
      const f32x16 p0 = mfma_fp8(a, w0, zero);
      const f32x16 p1 = mfma_fp8(a, w1, zero);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][r] = __builtin_fmaf(c0v[r], p0[r], acc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][r] = __builtin_fmaf(c1v[r], p1[r], acc[1][r]);
    }
  };
  for (int i = tid; i < GPS * BM; i += 512) zsc[i] = 0;
  StageRegs r0s, r1s;
  load_stage(rw, 0, G, tid, r0s);
  load_stage(rw, GPS, G, tid, r1s);
  store_stage(lds[0], tid, r0s, 0, G);
  __syncthreads();
  load_stage(rw, 2 * GPS, G, tid, r0s);
  for (int s = 0; s < S; s += 2) {
    // lds[0] holds stage s, r1s stage s+1, r0s stage s+2 (in flight)
    compute(lds[0]);
    store_stage(lds[1], tid, r1s, (s + 1) * GPS, G);
    __syncthreads();
    load_stage(rw, (s + 3) * GPS, G, tid, r1s);
    if (s + 1 >= S) break;
    compute(lds[1]);
    store_stage(lds[0], tid, r0s, (s + 2) * GPS, G);
    __syncthreads();
    load_stage(rw, (s + 4) * GPS, G, tid, r0s);
  }

  if constexpr (GU) {
    // g, u of column col for routed row `row`; c_g lacks the folded 2^12
    const float gs = *p.Sx * p.Sw13[e] * 4096.0f, Sh = *p.Sh;
    const int col = c0 + wn * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 32 + acc_row(r, lane);
      const float gv = acc[0][r] * gs, uv = acc[1][r] * gs;
      const float hv = (gv / (1.0f + expf(-gv))) * uv;
      // NVFP4 group of 16 columns: lanes l32 ^ 1, 2, 4, 8 of the same half
      float amax = fabsf(hv);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const uint32_t sb = f32_to_e4m3_rne_sat(amax / 6.0f / Sh);
      const float d = e4m3_to_f32(sb) * Sh;
      const uint32_t code = (sb & 0x7Fu) != 0u ? f32_to_e2m1_rne_sat(hv / d) : 0u;
      const uint32_t pair = code | (__shfl_xor(code, 1, 64) << 4);   // (even, odd) column pair
      if (row < nrows && (l32 & 1) == 0) {
        const int64_t srow = r0 + row;
        hq[srow * (I / 2) + col / 2] = (uint8_t)pair;
        if ((l32 & 15) == 0) hs[srow * (I / 16) + col / 16] = (uint8_t)sb;
        if (p.dbg_h) {
          uint8_t *d8 = p.dbg_h + (int64_t)sorted[srow] * (I / 2 + I / 16);
          d8[col / 2] = (uint8_t)pair;
          if ((l32 & 15) == 0) d8[I / 2 + col / 16] = (uint8_t)sb;
        }
      }
    }
  } else {
    if (tid < BM) s_w[tid] = wv;
    __syncthreads();
    const float gs = *p.Sh * p.Sw2[e] * 4096.0f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = c0 + (j ? ob1 : ob0) + l32;
      if (n >= H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 32 + acc_row(r, lane);
        if (row < nrows) y[(int64_t)(r0 + row) * H + n] = acc[j][r] * gs * s_w[row];
      }
    }
  }
}

}  // namespace

hipError_t launch_moe4_gemms(const Moe4Args &p, const int32_t *meta, const int32_t *sorted,
                             const float *wsorted, const int32_t *tile_e, const int32_t *tile_r,
                             const int32_t *tile_n, int maxtiles, uint8_t *hq, uint8_t *hs,
                             float *y, hipStream_t stream) {
  hipLaunchKernelGGL(k4_gemm<true>, dim3(p.I / 64, maxtiles), dim3(512), 0, stream, p, meta,
                     sorted, wsorted, tile_e, tile_r, tile_n, hq, hs, y);
  hipLaunchKernelGGL(k4_gemm<false>, dim3((p.H + BN - 1) / BN, maxtiles), dim3(512), 0, stream,
                     p, meta, sorted, wsorted, tile_e, tile_r, tile_n, hq, hs, y);
  return hipGetLastError();
}

}  // namespace mg
