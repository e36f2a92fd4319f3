// gemm_w4a8_tile.hip -- W4A8 (FP8 E4M3 per-token activations under NVFP4
// weights) for more than 32 tokens, through the exact E4M3 route of the
// metrale_circuit hardware::exec documentation (exec_of: NVFP4 weights under
// FP8 activations take the exact route):
//
//   * weight codes -> E4M3 by the E2M1 -> E4M3 bit identity (value x 2^-6);
//   * one v_mfma_f32_32x32x16_fp8_fp8 per 16-element group, zero accumulator;
//   * acc = fma(64 * s_w[n,g], P_g, acc) in FP32, groups in ascending K;
//   * epilogue: acc * a_tok[m] * S_w.
//
// With many tokens the per-group FMAs, not the weight stream, bound the
// operation, so it is tiled like the W4A4 kernel: 128 tokens x 128 weight
// rows per workgroup (8 waves, 4 x 2, wave tile 32 x 64), K staged through LDS
// 64 elements (4 groups) at a time, double-buffered, global loads two stages
// ahead in registers.  Tokens go to LDS as loaded, their bytes permuted into
// the order of the converted codes; weight codes are converted when written
// to LDS and their group scales decoded to FP32 (times 64) then.  A weight
// row's scale is one value per lane (the lane's output column), so the group
// step is one FMA per accumulator element and no MFMA.  K is split over ks
// workgroups (each a run of whole stages): FP32 partials, summed in split
// order by the decode path's reduction kernel.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int GPS = 4;        // groups (of 16 K-elements) per LDS stage

// byte offset of the 8 E4M3 values (K-elements 8h..8h+7 of group g) of tile
// row `row` in a stage: each (32-row block, group) is one 512-byte MFMA
// operand, lane (h, row % 32) at 8 * (32 h + row % 32)
__device__ __forceinline__ int coff(int row, int g, int h) {
  return ((((row >> 5) * GPS + g) * 64) + h * 32 + (row & 31)) * 8;
}

struct Stage {
  uint8_t code[2][BM * GPS * 16];   // tokens, weights: E4M3 in operand order
  float sw[GPS][BN];                // weight group scales x 64, [group][row]
};

// Every thread stages the same share of a stage (row tid / 4, group tid % 4
// of each operand), so no wave carries more of the conversion than another.
struct StageRegs {
  u32x4 a;         // one group (16 values) of one token row
  u32x2 w;         // the 16 codes of that group of one weight row
  uint32_t s;      // that weight row's scale byte of the group
};

// Global loads of one stage: addresses clamped in bounds, nothing selected
// on the data here (the stage store masks), so no load waits early.
__device__ __forceinline__ void load_stage(const W4A8Args &p, int m0, int n0, int g0, int G,
                                           int tid, StageRegs &r) {
  {
    const int row = tid >> 2, g = g0 + (tid & 3);
    int m = m0 + row;
    m = m < p.M ? m : p.M - 1;
    const int gs = g < G ? g : G - 1;
    r.a = *(const u32x4 *)(p.aq + (int64_t)m * p.K + (int64_t)gs * 16);
  }
  {
    const int row = tid >> 2, g = g0 + (tid & 3);
    int n = n0 + row;
    n = n < p.N ? n : p.N - 1;
    const int gs = g < G ? g : G - 1;
    r.w = *(const u32x2 *)(p.wq + (int64_t)n * (p.K / 2) + (int64_t)gs * 8);
    r.s = p.ws[(int64_t)n * (p.K / 16) + gs];
  }
}

// Stage g0 to LDS: tokens permuted, codes converted, scales decoded; groups
// at or past gend zeroed (tokens, codes and scales).
__device__ __forceinline__ void store_stage(Stage &s, int tid, const StageRegs &r, int g0, int gend) {
  {
    const int row = tid >> 2, g = tid & 3;
    const u32x4 v = g0 + g < gend ? r.a : u32x4{0, 0, 0, 0};
    *(uint64_t *)(s.code[0] + coff(row, g, 0)) = e4m3x8_even_odd((uint64_t)v[0] | ((uint64_t)v[1] << 32));
    *(uint64_t *)(s.code[0] + coff(row, g, 1)) = e4m3x8_even_odd((uint64_t)v[2] | ((uint64_t)v[3] << 32));
  }
  {
    const int row = tid >> 2, g = tid & 3;
    const bool in = g0 + g < gend;
    const u32x2 v = in ? r.w : u32x2{0, 0};
    // dwords: (group g, half 0) (g, 1)
    *(uint64_t *)(s.code[1] + coff(row, g, 0)) = nvfp4x8_to_e4m3x8(v[0]);
    *(uint64_t *)(s.code[1] + coff(row, g, 1)) = nvfp4x8_to_e4m3x8(v[1]);
    s.sw[g][row] = in ? e4m3_x64_to_f32_nan(r.s & 0xFFu) : 0.0f;
  }
}

__global__ __launch_bounds__(512, 2) void w4a8_tile_kernel(W4A8Args p, int ks, int gpw, float *part) {
  __shared__ __attribute__((aligned(16))) Stage lds[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int tile = blockIdx.x % (tiles_m * tiles_n), kc = blockIdx.x / (tiles_m * tiles_n);
  const int m0 = (tile % tiles_m) * BM, n0 = (tile / tiles_m) * BN;
  const int G = p.K / 16;
  const int gbeg = kc * gpw, gend = gbeg + gpw < G ? gbeg + gpw : G;   // this split's groups
  const int S = (gend - gbeg + GPS - 1) / GPS;

  f32x16 acc[2] = {f32x16{0}, f32x16{0}};
  const f32x16 zero = {0};

  auto compute = [&](const Stage &cur) {
    const uint8_t *pa = cur.code[0] + coff(wm * 32, 0, 0) + 8 * lane;
    const uint8_t *pw0 = cur.code[1] + coff(wn * 64, 0, 0) + 8 * lane;
    const uint8_t *pw1 = cur.code[1] + coff(wn * 64 + 32, 0, 0) + 8 * lane;
    const float *ps = cur.sw[0] + wn * 64 + l32;
#pragma unroll 1
    for (int g = 0; g < GPS; ++g) {
      const uint64_t a = *(const uint64_t *)(pa + 512 * g);
      const uint64_t w0 = *(const uint64_t *)(pw0 + 512 * g), w1 = *(const uint64_t *)(pw1 + 512 * g);
      const float s0 = ps[BN * g], s1 = ps[BN * g + 32];
      const f32x16 p0 = mfma_fp8(a, w0, zero);
      const f32x16 p1 = mfma_fp8(a, w1, zero);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][r] = __builtin_fmaf(s0, p0[r], acc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][r] = __builtin_fmaf(s1, p1[r], acc[1][r]);
    }
  };
  StageRegs r0, r1;
  load_stage(p, m0, n0, gbeg, G, tid, r0);
  load_stage(p, m0, n0, gbeg + GPS, G, tid, r1);
  store_stage(lds[0], tid, r0, gbeg, gend);
  __syncthreads();
  load_stage(p, m0, n0, gbeg + 2 * GPS, G, tid, r0);
  for (int s = 0; s < S; s += 2) {
    // lds[0] holds stage s, r1 stage s+1, r0 stage s+2 (in flight)
    compute(lds[0]);
    store_stage(lds[1], tid, r1, gbeg + (s + 1) * GPS, gend);
    __syncthreads();
    load_stage(p, m0, n0, gbeg + (s + 3) * GPS, G, tid, r1);
    if (s + 1 >= S) break;
    compute(lds[1]);
    store_stage(lds[0], tid, r0, gbeg + (s + 2) * GPS, gend);
    __syncthreads();
    load_stage(p, m0, n0, gbeg + (s + 4) * GPS, G, tid, r0);
  }

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + l32;
    if (n >= p.N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * 32 + acc_row(r, lane);
      if (m >= p.M) continue;
      if (ks > 1) {
        part[((int64_t)kc * p.M + m) * p.N + n] = acc[j][r];
      } else {
        const float v = acc[j][r] * (p.atok[m] * *p.Sw);
        if (p.out_f32)
          ((float *)p.C)[(int64_t)m * p.N + n] = v;
        else
          ((uint16_t *)p.C)[(int64_t)m * p.N + n] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

}  // namespace

// Split of K for the tile kernel: at most two workgroups per CU (256 CUs)
// in all, so the launch runs in one round, each split a run of whole stages.
void w4a8_tile_split(int64_t M, int64_t N, int64_t K, int &ks, int &gpw) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t G = K / 16, stages = (G + GPS - 1) / GPS;
  int64_t want = 512 / tiles;
  want = want < 1 ? 1 : (want > stages ? stages : want);
  const int64_t spw = (stages + want - 1) / want;             // stages per split
  gpw = (int)(spw * GPS);
  ks = (int)((G + gpw - 1) / gpw);
}

hipError_t launch_w4a8_tile(const W4A8Args &p, int ks, int gpw, float *part, hipStream_t stream) {
  const int64_t tiles = (int64_t)((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL(w4a8_tile_kernel, dim3((unsigned)(tiles * ks)), dim3(512), 0, stream, p, ks, gpw, part);
  return hipGetLastError();
}

}  // namespace mg
