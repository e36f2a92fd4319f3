// gemm_w4a4.hip -- NVFP4 x NVFP4 TN GEMM on gfx950 through the exact E4M3
// route of the metrale_circuit hardware::exec module description:
//
//   * both operands' E2M1 codes become E4M3 bytes by the mask-and-shift bit
//     identity (value x 2^-6), giving FP8 MFMA operands;
//   * one v_mfma_f32_32x32x16_fp8_fp8 per 16-element group with a zero
//     accumulator gives the group partial P'_g = 2^-12 P_g (exact in FP32);
//   * the group scale product c_g = s_a * s_w is formed exactly on the matrix
//     unit too: a second FP8 MFMA whose operands carry the raw E4M3 scale
//     bytes at K = 0 and zeros elsewhere (a NaN scale gives a NaN product);
//   * acc = fma(c_g, P'_g, acc) in FP32, groups in ascending K.  This is the
//     route's fma((64 s_a)(64 s_w), P'_g, acc) scaled by exactly 2^-12 at
//     every step, so every rounding is the same;
//   * epilogue: acc * (4096 S_a S_w), BF16 (nearest even) or FP32 store.
//
// Per 32x32 block and group the route costs two FP8 MFMAs and 16 FP32 FMAs,
// and the FMAs on the vector ALU are the bound.  Everything else is kept off
// that unit: codes are converted to E4M3 once, when a stage is written to LDS
// (not by every wave that reads them), scale bytes go to LDS untouched, LDS
// holds each (32-row block, group) operand contiguously in lane order (no
// bank conflicts), and global loads run two stages ahead of their use with no
// wait until the stage is written.
//
// Workgroup: 512 threads (8 waves, 4x2), tile 128 x 128, wave tile 32 x 64
// (1 x 2 MFMA blocks of 32 x 32, so 4 waves fit each SIMD).  K is staged
// through LDS 64 elements (4 groups) at a time, double-buffered.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int BM = 128, BN = 128;
constexpr int GPS = 4;        // groups (of 16 K-elements) per LDS stage
// byte offset of the 8 E4M3 codes (K-elements 8h..8h+7 of group g) of tile row
// `row` in a stage: each (32-row block, group) is one 512-byte MFMA operand,
// lane (h, row % 32) at 8 * (32 h + row % 32) -- a wave reads it contiguously
__device__ __forceinline__ int coff(int row, int g, int h) {
  return ((((row >> 5) * GPS + g) * 64) + h * 32 + (row & 31)) * 8;
}

// One stage: each operand's E4M3 codes in MFMA operand order (see coff), and
// each row's 4 raw group scale bytes, group-major, each widened to 8 bytes so
// one LDS read yields a whole MFMA operand (the byte at K = 0, zeros above).
struct Stage {
  uint8_t code[2][BM * GPS * 16];
  uint64_t sc[2][GPS * BM];   // [group][row]: raw E4M3 scale byte, zero-extended to 8 bytes
};

struct StageRegs {
  u32x4 code;      // 32 codes (groups 2q, 2q+1) of one row (threads < 256: A, else W)
  uint32_t s0, s1; // scale bytes of groups (0, 1) and (2, 3) of one row, as loaded
};

// Global loads of one stage.  Every thread issues the same loads with no
// data-dependent branch or select, so nothing waits for them here: the data
// is masked when the stage is written to LDS.  (Threads 256..511 repeat the
// scale loads of threads 0..255; only the latter store them.)
__device__ __forceinline__ void load_stage(const W4A4Args &p, int m0, int n0, int g0, int G,
                                           int tid, StageRegs &r) {
  const int64_t rowb = p.K / 2, rows = p.K / 16;
  {
    const int row = (tid & 255) >> 1, q = tid & 1;
    const int op = tid >> 8;
    const uint8_t *base = op == 0 ? p.aq : p.wq;
    const int R = op == 0 ? p.M : p.N, o = op == 0 ? m0 : n0;
    const int g = g0 + 2 * q;               // G is even (K % 32 == 0): g < G covers g + 1
    int grow = o + row;
    grow = grow < R ? grow : R - 1;
    const int gs = g < G ? g : G - 2;       // in-bounds address
    r.code = *(const u32x4 *)(base + (int64_t)grow * rowb + (int64_t)gs * 8);
  }
  {
    const int op = (tid >> 7) & 1, srow = tid & 127;
    const uint8_t *base = op == 0 ? p.as : p.ws;
    const int R = op == 0 ? p.M : p.N, o = op == 0 ? m0 : n0;
    int grow = o + srow;
    grow = grow < R ? grow : R - 1;
    const uint16_t *s16 = (const uint16_t *)(base + (int64_t)grow * rows);
    r.s0 = s16[(g0 < G ? g0 : G - 2) >> 1];
    r.s1 = s16[(g0 + 2 < G ? g0 + 2 : G - 2) >> 1];
  }
}

// Stage g0 to LDS: codes converted to E4M3, groups at or past G zeroed.
__device__ __forceinline__ void store_stage(Stage &s, int tid, const StageRegs &r, int g0, int G) {
  {
    const int row = (tid & 255) >> 1, q = tid & 1;
    const int op = tid >> 8;
    const u32x4 v = g0 + 2 * q < G ? r.code : u32x4{0, 0, 0, 0};
    // dwords: (group 2q, half 0) (2q, 1) (2q+1, 0) (2q+1, 1)
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

__global__ __launch_bounds__(512, 2) void w4a4_fp8route_kernel(W4A4Args p) {
  __shared__ __attribute__((aligned(16))) Stage lds[2];
  __shared__ uint64_t zsc[GPS * BM];   // zeros: the A-side scale operand of lanes h = 1

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, h = lane >> 5;
  int tm, tn;
  xcd_tile(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  const int n0 = tn * BN, m0 = tm * BM;
  const int G = p.K / 16;
  const int S = (G + GPS - 1) / GPS;

  f32x16 acc[2] = {f32x16{0}, f32x16{0}};
  const f32x16 zero = {0};

  // global loads run two stages ahead of their LDS store (a two-deep ring of
  // register buffers; loads past the last stage are clamped and masked)
  auto compute = [&](const Stage &cur) {
    const uint8_t *pa = cur.code[0] + coff(wm * 32, 0, 0) + 8 * lane;
    const uint8_t *pw0 = cur.code[1] + coff(wn * 64, 0, 0) + 8 * lane;
    const uint8_t *pw1 = cur.code[1] + coff(wn * 64 + 32, 0, 0) + 8 * lane;
    // scale operands: lane (row, h = 0) holds its row's scale byte at K = 0 and
    // zeros elsewhere; on the A side lanes h = 1 read zeros, so the K = 16
    // product is exactly s_a * s_w (a NaN scale still yields NaN)
    const uint64_t *psa = (h ? zsc : cur.sc[0]) + wm * 32 + l32;
    const uint64_t *psw = cur.sc[1] + wn * 64 + l32;
#pragma unroll 1
    for (int g = 0; g < GPS; ++g) {
      const uint64_t a = *(const uint64_t *)(pa + 512 * g);
      const uint64_t w0 = *(const uint64_t *)(pw0 + 512 * g), w1 = *(const uint64_t *)(pw1 + 512 * g);
      const uint64_t sa = psa[BM * g], sw0 = psw[BM * g], sw1 = psw[BM * g + 32];
      const f32x16 c0 = mfma_fp8(sa, sw0, zero);
      const f32x16 c1 = mfma_fp8(sa, sw1, zero);
      const f32x16 p0 = mfma_fp8(a, w0, zero);
      const f32x16 p1 = mfma_fp8(a, w1, zero);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][r] = __builtin_fmaf(c0[r], p0[r], acc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][r] = __builtin_fmaf(c1[r], p1[r], acc[1][r]);
    }
  };
  for (int i = tid; i < GPS * BM; i += 512) zsc[i] = 0;
  StageRegs r0, r1;
  load_stage(p, m0, n0, 0, G, tid, r0);
  load_stage(p, m0, n0, GPS, G, tid, r1);
  store_stage(lds[0], tid, r0, 0, G);
  __syncthreads();
  load_stage(p, m0, n0, 2 * GPS, G, tid, r0);
  for (int s = 0; s < S; s += 2) {
    // lds[0] holds stage s, r1 stage s+1, r0 stage s+2 (in flight)
    compute(lds[0]);
    store_stage(lds[1], tid, r1, (s + 1) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 3) * GPS, G, tid, r1);
    if (s + 1 >= S) break;
    compute(lds[1]);
    store_stage(lds[0], tid, r0, (s + 2) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 4) * GPS, G, tid, r0);
  }

  const float gs = *p.Sa * *p.Sw * 4096.0f;  // c_g lacks the folded 2^6 * 2^6
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn * 64 + j * 32 + l32;
    if (col >= p.N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 32 + acc_row(r, lane);
      if (row >= p.M) continue;
      const float v = acc[j][r] * gs;
      if (p.out_f32)
        ((float *)p.C)[(int64_t)row * p.N + col] = v;
      else
        ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// The same route on a 256 x 256 tile (M and N above 128): 512 threads (8
// waves, 4 x 2), wave tile 64 x 128 (2 x 4 blocks of 32 x 32).  Per stage a
// thread converts 32 codes of A and 32 of W, which now serve a wave's 8
// blocks per group instead of 2, and a wave reads 2 A and 4 W code operands
// and 2 + 4 scale operands per group for 8 blocks (12 LDS reads, half of the
// 128 x 128 tile's per block).  One workgroup per CU (2 waves per SIMD; the
// accumulators of 8 blocks take 128 registers).  Every FP32 rounding is the
// 128 x 128 kernel's (the same group terms in the same order).
//
// Scale operands here come from one word per row and stage: a row's four
// group scale bytes at K = 0..3 (zeros above).  A W-side lane passes its
// row's word whole; an A-side lane passes its row's word masked to group g's
// byte (lanes h = 1, K = 8..15: zero).  The K = 16 MFMA then sums one nonzero
// product, s_a * s_w of group g, exactly.  The other W bytes meet zeros; only
// a NaN among them changes the sum (to NaN), and that byte makes its whole
// output column NaN anyway.  This reads one scale word per block and stage
// instead of one 8-byte operand per block and group (LDS reads per stage and
// wave: 39 instead of 64 in the 224-wide kernel).
namespace big {

constexpr int BM = 256, BN = 256;
constexpr int GPS = 4;
__device__ __forceinline__ int coff(int row, int g, int h) {
  return ((((row >> 5) * GPS + g) * 64) + h * 32 + (row & 31)) * 8;
}
struct Stage {
  uint8_t code[2][BM * GPS * 16];   // A, W codes as E4M3 in MFMA operand order
  uint64_t sc[2][BM];               // [row]: the 4 groups' raw scale bytes at K = 0..3, zeros above
};
struct StageRegs {
  u32x4 a, w;        // 32 codes of one A row and one W row (groups 2q, 2q+1)
  uint32_t s0, s1;   // scale bytes of groups (0, 1) and (2, 3) of one row
};

__device__ __forceinline__ void load_stage(const W4A4Args &p, int m0, int n0, int g0, int G,
                                           int tid, StageRegs &r) {
  const int64_t rowb = p.K / 2, rows = p.K / 16;
  const int row = tid >> 1, q = tid & 1;
  const int g = g0 + 2 * q;
  const int gs = g < G ? g : G - 2;          // in-bounds address (G even)
  {
    const int ga = m0 + row < p.M ? m0 + row : p.M - 1;
    const int gw = n0 + row < p.N ? n0 + row : p.N - 1;
    r.a = *(const u32x4 *)(p.aq + (int64_t)ga * rowb + (int64_t)gs * 8);
    r.w = *(const u32x4 *)(p.wq + (int64_t)gw * rowb + (int64_t)gs * 8);
  }
  {
    // threads 0..255 fetch A rows' scales, 256..511 W rows'
    const int op = tid >> 8, srow = tid & 255;
    const uint8_t *base = op == 0 ? p.as : p.ws;
    const int R = op == 0 ? p.M : p.N, o = op == 0 ? m0 : n0;
    const int grow = o + srow < R ? o + srow : R - 1;
    const uint16_t *s16 = (const uint16_t *)(base + (int64_t)grow * rows);
    r.s0 = s16[(g0 < G ? g0 : G - 2) >> 1];
    r.s1 = s16[(g0 + 2 < G ? g0 + 2 : G - 2) >> 1];
  }
}

__device__ __forceinline__ void store_codes(uint8_t *c, int row, int q, u32x4 v) {
  const uint64_t e0 = nvfp4x8_to_e4m3x8(v[0]), e1 = nvfp4x8_to_e4m3x8(v[1]);
  const uint64_t e2 = nvfp4x8_to_e4m3x8(v[2]), e3 = nvfp4x8_to_e4m3x8(v[3]);
  *(uint64_t *)(c + coff(row, 2 * q, 0)) = e0;
  *(uint64_t *)(c + coff(row, 2 * q, 1)) = e1;
  *(uint64_t *)(c + coff(row, 2 * q + 1, 0)) = e2;
  *(uint64_t *)(c + coff(row, 2 * q + 1, 1)) = e3;
}

__device__ __forceinline__ void store_stage(Stage &s, int tid, const StageRegs &r, int g0, int G) {
  const int row = tid >> 1, q = tid & 1;
  const bool in = g0 + 2 * q < G;
  store_codes(s.code[0], row, q, in ? r.a : u32x4{0, 0, 0, 0});
  store_codes(s.code[1], row, q, in ? r.w : u32x4{0, 0, 0, 0});
  const uint32_t w = (g0 < G ? r.s0 : 0u) | ((g0 + 2 < G ? r.s1 : 0u) << 16);
  s.sc[tid >> 8][tid & 255] = w;   // zero-extended: K = 4..7 of the operand read as 0
}

__global__ __launch_bounds__(512, 1) void w4a4_fp8route_big(W4A4Args p) {
  __shared__ __attribute__((aligned(16))) Stage lds[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, h = lane >> 5;
  int tm, tn;
  xcd_tile(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  const int n0 = tn * BN, m0 = tm * BM;
  const int G = p.K / 16;
  const int S = (G + GPS - 1) / GPS;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};
  const f32x16 zero = {0};

  // scale operands (see scale_ops): A-side lanes take their row's word
  // masked to group g's byte (lanes h = 1: zero), W-side lanes their row's
  // whole word, so the K = 16 product is exactly s_a * s_w of group g
  uint32_t amask[GPS];
#pragma unroll
  for (int g = 0; g < GPS; ++g) amask[g] = h ? 0u : 0xFFu << (8 * g);
  auto compute = [&](const Stage &cur) {
    const uint8_t *pa = cur.code[0] + coff(wm * 64, 0, 0) + 8 * lane;
    const uint8_t *pw = cur.code[1] + coff(wn * 128, 0, 0) + 8 * lane;
    uint32_t saw[2];
    uint64_t sw[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) saw[i] = (uint32_t)cur.sc[0][wm * 64 + 32 * i + l32];
#pragma unroll
    for (int j = 0; j < 4; ++j) sw[j] = cur.sc[1][wn * 128 + 32 * j + l32];
    // the next block's scale product is issued after the current block's
    // P'_g MFMA, as in the 224-wide kernel
    f32x16 cn = mfma_fp8(saw[0] & amask[0], sw[0], zero);
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      uint64_t a[2], w[4], sa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *(const uint64_t *)(pa + (i * GPS + g) * 512);
        sa[i] = saw[i] & amask[g];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = *(const uint64_t *)(pw + (j * GPS + g) * 512);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int i = b >> 2, j = b & 3;
        const f32x16 c = cn;
        __builtin_amdgcn_s_setprio(1);   // see the 224-wide kernel below
        const f32x16 pp = mfma_fp8(a[i], w[j], zero);
        __builtin_amdgcn_sched_barrier(0);
        if (b < 7)
          cn = mfma_fp8(sa[(b + 1) >> 2], sw[(b + 1) & 3], zero);
        else if (g + 1 < GPS)
          cn = mfma_fp8(saw[0] & amask[g + 1], sw[0], zero);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(c[r], pp[r], acc[i][j][r]);
      }
    }
  };
  StageRegs r0, r1;
  load_stage(p, m0, n0, 0, G, tid, r0);
  load_stage(p, m0, n0, GPS, G, tid, r1);
  store_stage(lds[0], tid, r0, 0, G);
  __syncthreads();
  load_stage(p, m0, n0, 2 * GPS, G, tid, r0);
  for (int s = 0; s < S; s += 2) {
    // lds[0] holds stage s, r1 stage s+1, r0 stage s+2 (in flight)
    compute(lds[0]);
    store_stage(lds[1], tid, r1, (s + 1) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 3) * GPS, G, tid, r1);
    if (s + 1 >= S) break;
    compute(lds[1]);
    store_stage(lds[0], tid, r0, (s + 2) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 4) * GPS, G, tid, r0);
  }

  const float gsc = *p.Sa * *p.Sw * 4096.0f;  // c_g lacks the folded 2^6 * 2^6
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 128 + j * 32 + l32;
    if (col >= p.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
        const float v = acc[i][j][r] * gsc;
        if (p.out_f32)
          ((float *)p.C)[(int64_t)row * p.N + col] = v;
        else
          ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
      }
  }
}

// The same route on a 256 x 224 tile: 8 waves (8 x 1) of 32 x 224 (1 x 7
// blocks, 112 accumulator registers); per group a wave reads 1 A and 7 W
// code operands for 7 blocks, and per stage 1 + 7 scale words.  For shapes whose
// 256 x 256 grid leaves a partial last round (N = 5376 and M = 8192: 672
// tiles = 2.6 rounds of 256 CUs) the 224-wide grid can fill whole rounds
// (768 tiles = 3 rounds, each tile 7/8 of the work).  Staging is the
// 256 x 256 kernel's (W rows 224..255 are staged and not read).  Each
// block's two MFMAs are issued at raised wave priority: the wave that
// reaches its MFMAs gets the issue slot ahead of the other wave's FMAs on
// the same SIMD, so the matrix unit and the FP32 FMAs overlap more (645-650
// against 622-627 TFLOP/s at the headline shape without it).  The scale
// product of the next block is issued right after the current block's P'_g
// MFMA (16 more registers, 244 in all), so it runs on the matrix unit while
// the wave's own FMAs of the current block issue (652-653 against 647).  No
// scheduling barrier separates the groups of a stage, so the next group's
// operand reads are issued under the current group's MFMAs and FMAs
// (704 against 656 TFLOP/s, same registers, output bit-identical).
constexpr int BN7 = 224;

__global__ __launch_bounds__(512, 1) void w4a4_fp8route_n224(W4A4Args p) {
  __shared__ __attribute__((aligned(16))) Stage lds[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  int tm, tn;
  xcd_tile(blockIdx.x, (p.M + BM - 1) / BM, (p.N + BN7 - 1) / BN7, tm, tn);
  const int n0 = tn * BN7, m0 = tm * BM;
  const int G = p.K / 16;
  const int S = (G + GPS - 1) / GPS;

  f32x16 acc[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) acc[j] = f32x16{0};
  const f32x16 zero = {0};

  uint32_t amask[GPS];   // as in the 256 x 256 kernel
#pragma unroll
  for (int g = 0; g < GPS; ++g) amask[g] = h ? 0u : 0xFFu << (8 * g);
  auto compute = [&](const Stage &cur) {
    const uint8_t *pa = cur.code[0] + coff(wave * 32, 0, 0) + 8 * lane;
    const uint8_t *pw = cur.code[1] + 8 * lane;
    const uint32_t saw = (uint32_t)cur.sc[0][wave * 32 + l32];
    uint64_t sw[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) sw[j] = cur.sc[1][32 * j + l32];
    f32x16 cn = mfma_fp8(saw & amask[0], sw[0], zero);
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      const uint64_t a = *(const uint64_t *)(pa + g * 512);
      uint64_t w[7];
#pragma unroll
      for (int j = 0; j < 7; ++j) w[j] = *(const uint64_t *)(pw + (j * GPS + g) * 512);
#pragma unroll
      for (int j = 0; j < 7; ++j) {
        const f32x16 c = cn;
        __builtin_amdgcn_s_setprio(1);
        const f32x16 pp = mfma_fp8(a, w[j], zero);
        __builtin_amdgcn_sched_barrier(0);
        if (j < 6)
          cn = mfma_fp8(saw & amask[g], sw[j + 1], zero);
        else if (g + 1 < GPS)
          cn = mfma_fp8(saw & amask[g + 1], sw[0], zero);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = __builtin_fmaf(c[r], pp[r], acc[j][r]);
      }
    }
  };
  StageRegs r0, r1;
  load_stage(p, m0, n0, 0, G, tid, r0);
  load_stage(p, m0, n0, GPS, G, tid, r1);
  store_stage(lds[0], tid, r0, 0, G);
  __syncthreads();
  load_stage(p, m0, n0, 2 * GPS, G, tid, r0);
  for (int s = 0; s < S; s += 2) {
    // lds[0] holds stage s, r1 stage s+1, r0 stage s+2 (in flight)
    compute(lds[0]);
    store_stage(lds[1], tid, r1, (s + 1) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 3) * GPS, G, tid, r1);
    if (s + 1 >= S) break;
    compute(lds[1]);
    store_stage(lds[0], tid, r0, (s + 2) * GPS, G);
    __syncthreads();
    load_stage(p, m0, n0, (s + 4) * GPS, G, tid, r0);
  }

  const float gsc = *p.Sa * *p.Sw * 4096.0f;  // c_g lacks the folded 2^6 * 2^6
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int col = n0 + j * 32 + l32;
    if (col >= p.N) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wave * 32 + acc_row(r, lane);
      if (row >= p.M) continue;
      const float v = acc[j][r] * gsc;
      if (p.out_f32)
        ((float *)p.C)[(int64_t)row * p.N + col] = v;
      else
        ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

}  // namespace big

}  // namespace

static int w4a4_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return n;
}

hipError_t launch_w4a4(const W4A4Args &p, hipStream_t stream) {
  // the 256 x 256 tile for large products; small ones keep the 128 x 128
  // tile (less padding, more workgroups)
  if (p.M > 128 && p.N > 128) {
    // tile width 256 or 224: whichever needs fewer rounds x width (one
    // workgroup per CU, a round's time proportional to the width)
    const int64_t tm = (p.M + big::BM - 1) / big::BM, cus = w4a4_cus();
    const int64_t t8 = tm * ((p.N + big::BN - 1) / big::BN), t7 = tm * ((p.N + big::BN7 - 1) / big::BN7);
    if ((t7 + cus - 1) / cus * 7 < (t8 + cus - 1) / cus * 8) {
      hipLaunchKernelGGL(big::w4a4_fp8route_n224, dim3((unsigned)t7), dim3(512), 0, stream, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(big::w4a4_fp8route_big, dim3((unsigned)t8), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM));
  hipLaunchKernelGGL(w4a4_fp8route_kernel, grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mg
