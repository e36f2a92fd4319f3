// gemm_bf16.hip -- BF16-activation TN GEMMs on the gfx950 BF16 MFMA:
//   W16A16: C = A . W^T, both BF16 (the H3 FFN down projection of RL-Kernel
//           PR #535: BF16 MMA tiles, FP32 accumulation, BF16 epilogue);
//   W4A16:  NVFP4 weights widened to BF16 (hardware::exec module description:
//           BF16 activations take the BF16 MMA, the weight widened in
//           registers).  Each weight element e2m1 x e4m3 is exact in BF16 (at
//           most 6 significant bits, exponent within range), so the products
//           are the declared ones; the FP32 tensor scale S_w is applied in the
//           epilogue (an arbitrary FP32 value would not be exact in BF16).
//
// Workgroup: 512 threads (8 waves, 4 along M x 2 along N), tile 256 x 128,
// K staged 64 at a time; wave tile 64 x 64 = 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16; one workgroup per CU.
//   * BF16 operands go from global memory straight into LDS (16-byte
//     global_load_lds: lane i's bytes land at the instruction's LDS base +
//     16 i), three stages deep, so two stages are in flight while one is
//     computed and no registers are spent on staging.  The lane -> global
//     chunk assignment realises the XOR swizzle of the LDS rows (see swz), so
//     the MFMA fragment reads (32 rows x one chunk) hit distinct banks.
//   * NVFP4 weights (W4A16) are loaded to registers one stage ahead, widened
//     to BF16 and written to the same LDS layout.
//   * Tiles are assigned XCD by XCD (see xcd_tile) so the workgroups sharing
//     an L2 share A and W panels.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int NTHR = 512;            // 8 waves
constexpr int ROWB = BK * 2;         // bytes per LDS row (64 BF16)
constexpr int STAGE_A = BM * ROWB, STAGE_W = BN * ROWB;


// 16-byte chunk `chunk` of tile row `row`: rows are 128 bytes, and the chunk
// is XOR-ed with (row / 2) % 8, so any 16 consecutive rows read at one chunk
// index cover 16 distinct 16-byte bank groups of the 256-byte bank window.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// E2M1 code (low 4 bits) -> FP32 value
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t mag = c & 7u;
  // magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: exponent field 126 + (mag >> 1) for
  // mag >= 2, with mantissa bit (mag & 1); mag 1 is 0.5, mag 0 is 0
  uint32_t bits = mag >= 2u ? (((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22)
                            : (mag == 1u ? 0x3F000000u : 0u);
  bits |= (c & 8u) << 28;
  return __builtin_bit_cast(float, bits);
}

// Issue the direct-to-LDS loads of one BF16 operand tile (R rows x 64 K) at
// k0 into `lds`.  Each wave instruction fills 1 KB = 8 rows; lane i fills LDS
// position (row 8b + i / 8, slot i % 8), which holds global chunk
// slot ^ ((row / 2) % 8).  Rows past the matrix read its last row (never
// stored); chunks past K read the row's last chunk (zeroed by fix_k_tail).
template <int R>
__device__ __forceinline__ void dma_tile(const uint16_t *src, int rows, int K, int r0, int k0,
                                         uint8_t *lds, int wave, int lane) {
  constexpr int BLOCKS = R / 8;                 // 1 KB blocks
  constexpr int PER_WAVE = BLOCKS / (NTHR / 64);
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int b = wave * PER_WAVE + j;
    const int row = 8 * b + (lane >> 3), slot = lane & 7;
    const int chunk = slot ^ ((row >> 1) & 7);
    int grow = r0 + row;
    grow = grow < rows ? grow : rows - 1;
    int k = k0 + 8 * chunk;
    k = k < K ? k : K - 8;
    dma16(src + (int64_t)grow * K + k, lds + 1024 * b);
  }
}

// Zero the chunks of a staged tile that lie past K (only the last stage of a
// K that is not a multiple of 64 has any).
template <int R>
__device__ __forceinline__ void fix_k_tail(uint8_t *lds, int K, int k0, int tid) {
  for (int c = tid; c < R * 8; c += NTHR) {
    const int row = c >> 3, chunk = c & 7;
    if (k0 + 8 * chunk >= K) *(u32x4 *)(lds + swz(row, chunk)) = u32x4{0, 0, 0, 0};
  }
}

struct WqRegs {
  u32x4 codes;    // 32 codes (two groups) of one weight half-row (threads < 256)
  uint32_t sc;    // their two scale bytes
};

__device__ __forceinline__ void wq_load(const Bf16Args &p, int n0, int k0, int tid, WqRegs &r) {
  const uint8_t *wq = (const uint8_t *)p.w;
  const int row = (tid & 255) >> 1, half = tid & 1;
  int grow = n0 + row;
  grow = grow < p.N ? grow : p.N - 1;
  const int k = k0 + half * 32, kc = k < p.K ? k : p.K - 32;  // in-bounds address; data masked
  const u32x4 v = *(const u32x4 *)(wq + (int64_t)grow * (p.K / 2) + kc / 2);
  r.codes = k < p.K ? v : u32x4{0, 0, 0, 0};
  const uint32_t sv = *(const uint16_t *)(p.ws + (int64_t)grow * (p.K / 16) + kc / 16);
  r.sc = k < p.K ? sv : 0u;
}

// widen 32 codes (two groups) to BF16: value = e2m1 * e4m3(scale), exact
__device__ __forceinline__ void wq_store(uint8_t *lw, int tid, const WqRegs &r) {
  if (tid >= 256) return;
  const int row = tid >> 1, half = tid & 1;
  const float s0 = e4m3_to_f32(r.sc & 0xFFu), s1 = e4m3_to_f32((r.sc >> 8) & 0xFFu);
#pragma unroll
  for (int q = 0; q < 4; ++q) {      // 16 B of codes -> 4 chunks of 8 BF16
    const uint32_t word = r.codes[q];
    const float s = q < 2 ? s0 : s1;  // bytes 0..7: group 0, bytes 8..15: group 1
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (word >> (8 * b)) & 0xFFu;
      const float lo = e2m1_to_f32(byte & 15u) * s, hi = e2m1_to_f32(byte >> 4) * s;
      out[b] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
    }
    *(u32x4 *)(lw + swz(row, half * 4 + q)) = out;
  }
}

template <bool WQ>
__global__ __launch_bounds__(NTHR, 1) void bf16_gemm_kernel(Bf16Args p) {
  // the three ring slots are separate arrays so the compiler can tell the
  // loads landing in one slot from the reads of another (and does not wait
  // for loads it does not need)
  __shared__ __attribute__((aligned(1024))) uint8_t la0[STAGE_A], la1[STAGE_A], la2[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[STAGE_W], lw1[STAGE_W], lw2[STAGE_W];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int S = (p.K + BK - 1) / BK;
  // this workgroup's tile and K range: the first full_tiles workgroups take
  // whole tiles; each later one one of `split` K ranges (in stages) of the
  // remaining tiles, written as an FP32 partial tile
  int tile = blockIdx.x, s_lo = 0, s_hi = S;
  float *part = nullptr;
  if (!WQ && (int)blockIdx.x >= p.full_tiles) {
    const int u = blockIdx.x - p.full_tiles, sp = u % p.split;
    tile = p.full_tiles + u / p.split;
    s_lo = (int)((int64_t)S * sp / p.split);
    s_hi = (int)((int64_t)S * (sp + 1) / p.split);
    part = p.part + (int64_t)u * BM * BN;
  }
  int tm, tn;
  xcd_tile(tile, (p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  const int n0 = tn * BN, m0 = tm * BM;
  const uint16_t *wb = (const uint16_t *)p.w;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

  // loads of stage t into a ring slot (stages past the end reload the last
  // one: same addresses, never computed)
  // (t counts stages from s_lo; stages past the range reload its last one:
  // same addresses, never computed)
  auto issue = [&](int t, uint8_t *la, uint8_t *lw) {
    const int tt = s_lo + t < s_hi ? s_lo + t : s_hi - 1;
    dma_tile<BM>(p.a, p.M, p.K, m0, tt * BK, la, wave, lane);
    if (!WQ) dma_tile<BN>(wb, p.N, p.K, n0, tt * BK, lw, wave, lane);
  };
  // direct loads per thread per stage (A, then W unless it is NVFP4)
  constexpr int LOADS = BM / 8 / (NTHR / 64) + (WQ ? 0 : BN / 8 / (NTHR / 64));

  WqRegs wr;
  // one stage: stage s sits in (la, lw); stage s+2 is issued into (na, nw),
  // the slot stage s-1 used
  auto step = [&](int s, uint8_t *la, uint8_t *lw, uint8_t *na, uint8_t *nw) {
    __builtin_amdgcn_sched_barrier(0);
    if (WQ) {
      // W of stage s from registers (loaded a stage ahead); the slot was last
      // read by stage s - 3, which every wave finished before the previous barrier
      wq_store(lw, tid, wr);
      wq_load(p, n0, (s + 1) * BK, tid, wr);
    }
    // stage s has landed once at most stage s+1's loads are outstanding
    // (the W4A16 register loads of stage s+1 were issued after them); LDS
    // writes of this thread are complete once lgkmcnt is 0.  The barrier is
    // the bare s_barrier: a fenced one would wait for every load in flight.
    wait_vmcnt<WQ ? LOADS + 2 : LOADS>();
    if (s == S - 1 && p.K % BK != 0) {
      // every thread's loads of the stage have landed before any thread
      // zeroes chunks that another thread loaded
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      fix_k_tail<BM>(la, p.K, s * BK, tid);
      if (!WQ) fix_k_tail<BN>(lw, p.K, s * BK, tid);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + 2, na, nw);
    // operand fragments double-buffered: the reads of K-step kk+1 are in
    // flight while the MFMAs of step kk run
    u32x4 fa[2][2], fw[2][2];
    auto frag = [&](int kk, int b) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[b][i] = *(const u32x4 *)(la + swz(wm * 64 + i * 32 + l32, 2 * kk + h));
        fw[b][i] = *(const u32x4 *)(lw + swz(wn * 64 + i * 32 + l32, 2 * kk + h));
      }
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) frag(kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of the MFMAs
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[kk & 1][i], fw[kk & 1][j], acc[i][j]);
    }
  };
  if constexpr (WQ) {
    wq_load(p, n0, 0, tid, wr);
    issue(0, la0, lw0);
    issue(1, la1, lw1);
    // whole ring turns, then the last one or two stages: the loop has a single
    // exit, which keeps each accumulator in one set of registers
    const int full = S - S % 3;
    for (int s = 0; s < full; s += 3) {
      step(s, la0, lw0, la2, lw2);
      step(s + 1, la1, lw1, la0, lw0);
      step(s + 2, la2, lw2, la1, lw1);
    }
    if (S % 3 >= 1) step(full, la0, lw0, la2, lw2);
    if (S % 3 == 2) step(full + 1, la1, lw1, la0, lw0);
  } else {
    // BF16 x BF16, pipelined across stages: the MFMAs of a stage's last
    // K-step are issued after the wave has met the others at the barrier for
    // the next stage and read that stage's first fragments, so the barrier
    // and those reads overlap the MFMAs in flight.  Past that barrier no wave
    // reads the current slot any more, so it is refilled right away with the
    // stage three ahead: three stages are in flight in three slots.
    u32x4 fa[2][2], fw[2][2];
    auto frag = [&](const uint8_t *la, const uint8_t *lw, int kk, int b) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[b][i] = *(const u32x4 *)(la + swz(wm * 64 + i * 32 + l32, 2 * kk + h));
        fw[b][i] = *(const u32x4 *)(lw + swz(wn * 64 + i * 32 + l32, 2 * kk + h));
      }
    };
    auto mfmas = [&](int b) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[b][i], fw[b][j], acc[i][j]);
    };
    // make stage t's slot readable: its loads landed (one or two later
    // stages' loads may still be in flight), the K tail zeroed, every wave
    // past the barrier
    const int SL = s_hi - s_lo;   // stages of this workgroup's K range
    auto ready = [&](int t, uint8_t *la, uint8_t *lw, bool two_after) {
      if (two_after)
        wait_vmcnt<2 * LOADS>();
      else
        wait_vmcnt<LOADS>();
      if (s_lo + t == S - 1 && p.K % BK != 0) {
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        fix_k_tail<BM>(la, p.K, (s_lo + t) * BK, tid);
        fix_k_tail<BN>(lw, p.K, (s_lo + t) * BK, tid);
      }
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    };
    // stage s computed from (la, lw); stage s+1 waits in (na, nw)
    auto step2 = [&](int s, uint8_t *la, uint8_t *lw, uint8_t *na, uint8_t *nw) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < BK / 16) {
          frag(la, lw, kk + 1, (kk + 1) & 1);
        } else if (s + 1 < SL) {
          ready(s + 1, na, nw, false);
          __builtin_amdgcn_sched_barrier(0);
          issue(s + 3, la, lw);
          frag(na, nw, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas(kk & 1);
      }
    };
    issue(0, la0, lw0);
    issue(1, la1, lw1);
    issue(2, la2, lw2);
    ready(0, la0, lw0, true);
    frag(la0, lw0, 0, 0);
    const int full = SL - SL % 3;
    for (int s = 0; s < full; s += 3) {
      step2(s, la0, lw0, la1, lw1);
      step2(s + 1, la1, lw1, la2, lw2);
      step2(s + 2, la2, lw2, la0, lw0);
    }
    if (SL % 3 >= 1) step2(full, la0, lw0, la1, lw1);
    if (SL % 3 == 2) step2(full + 1, la1, lw1, la2, lw2);
  }
  wait_vmcnt<0>();

  const float gs = WQ ? *p.Sw : 1.0f;
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
        if (!WQ && part) {   // a K range of a split tile: FP32 partial, tile-local
          part[(row - m0) * BN + (col - n0)] = acc[i][j][r];
          continue;
        }
        const float v = WQ ? acc[i][j][r] * gs : acc[i][j][r];
        if (p.out_f32)
          ((float *)p.C)[(int64_t)row * p.N + col] = v;
        else
          ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

// BF16 x BF16 on a 256 x 256 tile: 8 waves (4 x 2) of 64 x 128 (2 x 4
// blocks, 128 accumulator registers).  A tile reads 256 + 256 rows per K
// stage for 2 * 256 * 256 * 64 flops (128 flops per byte, against 85 for
// 256 x 128), which halves the operand traffic from L2 per flop, and each
// wave reads 6 fragments per 8 MFMAs.  Two 64 KiB ring slots: stage s + 2 is
// requested right after the barrier that follows the last read of stage s,
// so one stage is in flight while the next is computed.  Same tail split as
// the 256 x 128 kernel.
namespace t256 {

constexpr int TBN = 256, TSW = TBN * ROWB;

// Byte offsets (from the matrix base moved to the stage's k0) of the rows
// and chunks one thread loads for an R-row tile, as dma_tile lays them out;
// valid while the tensor is under 4 GiB.
template <int R>
__device__ __forceinline__ void dma_offsets(int rows, int K, int r0, int wave, int lane,
                                            uint32_t (&off)[R / 64]) {
#pragma unroll
  for (int j = 0; j < R / 64; ++j) {
    const int row = 8 * (wave * (R / 64) + j) + (lane >> 3), slot = lane & 7;
    const int chunk = slot ^ ((row >> 1) & 7);
    int grow = r0 + row;
    grow = grow < rows ? grow : rows - 1;
    off[j] = (uint32_t)grow * (uint32_t)K * 2u + 16u * chunk;
  }
}
// dma_tile from those offsets; in the stage that crosses K (k0 + 64 > K) a
// chunk past K reads the row's last chunk instead (zeroed by fix_k_tail)
template <int R>
__device__ __forceinline__ void dma_tile_s(const uint16_t *src, int K, int k0,
                                           const uint32_t (&off)[R / 64], uint32_t lds, int wave,
                                           int lane) {
  const uint16_t *base = src + k0;
  const int kr = K - 8 - k0;   // element offset of the row's last chunk from k0
#pragma unroll
  for (int j = 0; j < R / 64; ++j) {
    uint32_t o = off[j];
    if (kr < BK - 8) {
      const int row = 8 * (wave * (R / 64) + j) + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      if (8 * chunk > kr) o = o - 16u * chunk + 2u * kr;
    }
    dma16_s(o, base, lds + 1024u * (wave * (R / 64) + j));
  }
}

__global__ __launch_bounds__(NTHR, 1) void bf16_gemm_256(Bf16Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t la0[STAGE_A], la1[STAGE_A];
  __shared__ __attribute__((aligned(1024))) uint8_t lw0[TSW], lw1[TSW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int S = (p.K + BK - 1) / BK;
  int tile = blockIdx.x, s_lo = 0, s_hi = S;
  float *part = nullptr;
  if ((int)blockIdx.x >= p.full_tiles) {
    const int u = blockIdx.x - p.full_tiles, sp = u % p.split;
    tile = p.full_tiles + u / p.split;
    s_lo = (int)((int64_t)S * sp / p.split);
    s_hi = (int)((int64_t)S * (sp + 1) / p.split);
    part = p.part + (int64_t)u * BM * TBN;
  }
  int tm, tn;
  xcd_tile(tile, (p.M + BM - 1) / BM, (p.N + TBN - 1) / TBN, tm, tn);
  const int n0 = tn * TBN, m0 = tm * BM;
  const uint16_t *wb = (const uint16_t *)p.w;
  const int SL = s_hi - s_lo;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};

  uint32_t offa[BM / 64], offw[TBN / 64];
  dma_offsets<BM>(p.M, p.K, m0, wave, lane, offa);
  dma_offsets<TBN>(p.N, p.K, n0, wave, lane, offw);
  auto issue = [&](int t, uint8_t *la, uint8_t *lw) {
    const int tt = s_lo + t < s_hi ? s_lo + t : s_hi - 1;
    dma_tile_s<BM>(p.a, p.K, tt * BK, offa, lds_addr(la), wave, lane);
    dma_tile_s<TBN>(wb, p.K, tt * BK, offw, lds_addr(lw), wave, lane);
  };
  constexpr int LOADS = BM / 8 / (NTHR / 64) + TBN / 8 / (NTHR / 64);
  u32x4 fa[2][2], fw[2][4];
  auto frag = [&](const uint8_t *la, const uint8_t *lw, int kk, int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      fa[b][i] = *(const u32x4 *)(la + swz(wm * 64 + i * 32 + l32, 2 * kk + h));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fw[b][j] = *(const u32x4 *)(lw + swz(wn * 128 + j * 32 + l32, 2 * kk + h));
  };
  auto mfmas = [&](int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[b][i], fw[b][j], acc[i][j]);
  };
  // stage t readable: its loads landed (one later stage's may be in flight),
  // the K tail zeroed, every wave past the barrier
  auto ready = [&](int t, uint8_t *la, uint8_t *lw, bool one_after) {
    if (one_after)
      wait_vmcnt<LOADS>();
    else
      wait_vmcnt<0>();
    if (s_lo + t == S - 1 && p.K % BK != 0) {
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      fix_k_tail<BM>(la, p.K, (s_lo + t) * BK, tid);
      fix_k_tail<TBN>(lw, p.K, (s_lo + t) * BK, tid);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };
  // stage s computed from (la, lw); stage s+1 waits in (na, nw); after the
  // barrier of stage s+1 no wave reads (la, lw) any more: stage s+2 goes there
  auto step2 = [&](int s, uint8_t *la, uint8_t *lw, uint8_t *na, uint8_t *nw) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < BK / 16) {
        frag(la, lw, kk + 1, (kk + 1) & 1);
      } else if (s + 1 < SL) {
        ready(s + 1, na, nw, false);
        __builtin_amdgcn_sched_barrier(0);
        issue(s + 2, la, lw);
        frag(na, nw, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(kk & 1);
    }
  };
  issue(0, la0, lw0);
  issue(1, la1, lw1);
  ready(0, la0, lw0, true);
  frag(la0, lw0, 0, 0);
  const int full = SL - SL % 2;
  for (int s = 0; s < full; s += 2) {
    step2(s, la0, lw0, la1, lw1);
    step2(s + 1, la1, lw1, la0, lw0);
  }
  if (SL % 2) step2(full, la0, lw0, la1, lw1);
  wait_vmcnt<0>();

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + l32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + acc_row(r, lane);
        if (row >= p.M) continue;
        if (part) {
          part[(row - m0) * TBN + (col - n0)] = acc[i][j][r];
          continue;
        }
        const float v = acc[i][j][r];
        if (p.out_f32)
          ((float *)p.C)[(int64_t)row * p.N + col] = v;
        else
          ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

}  // namespace t256

// the split tiles (BM x TN): C = sum of the tile's `split` FP32 partials in
// split order; a thread takes 8 consecutive elements of a row
template <int TN>
__global__ __launch_bounds__(256) void bf16_tail_sum(Bf16Args p) {
  const int tail = blockIdx.y, e = (blockIdx.x * 256 + threadIdx.x) * 8;   // element of the tile
  if (e >= BM * TN) return;
  int tm, tn;
  xcd_tile(p.full_tiles + tail, (p.M + BM - 1) / BM, (p.N + TN - 1) / TN, tm, tn);
  const int row = tm * BM + e / TN, col = tn * TN + e % TN;
  if (row >= p.M || col >= p.N) return;
  const float *src = p.part + (int64_t)tail * p.split * BM * TN + e;
  float v[8];
  {
    const f32x4 a = *(const f32x4 *)src, b = *(const f32x4 *)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = a[i], v[4 + i] = b[i];
  }
  for (int s = 1; s < p.split; ++s) {
    const float *q = src + (int64_t)s * BM * TN;
    const f32x4 a = *(const f32x4 *)q, b = *(const f32x4 *)(q + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] += a[i], v[4 + i] += b[i];
  }
  const int64_t o = (int64_t)row * p.N + col;
  if (col + 8 <= p.N && p.N % 8 == 0 && ((uintptr_t)p.C & 15) == 0) {   // whole and aligned
    if (p.out_f32) {
      *(f32x4 *)((float *)p.C + o) = f32x4{v[0], v[1], v[2], v[3]};
      *(f32x4 *)((float *)p.C + o + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
      *(u32x4 *)((uint16_t *)p.C + o) = w;
    }
    return;
  }
  for (int i = 0; i < 8 && col + i < p.N; ++i) {
    if (p.out_f32)
      ((float *)p.C)[o + i] = v[i];
    else
      ((uint16_t *)p.C)[o + i] = (uint16_t)f32_to_bf16_rne(v[i]);
  }
}

int cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return n;
}

// The grid runs one workgroup per CU, so T tiles take ceil(T / CUs) rounds.
// When the last round is partial, its R tiles can each be split into s K
// ranges (s R units of 1/s of a tile): the tail then takes ceil(s R / CUs) /
// s of a round, and the s R FP32 partial tiles are read back by a second
// kernel.  s (1..16, at least 4 stages per range) minimises the estimate
//   ceil(s R / CUs) / s * t_tile + s R * 128 KiB / (4 TB/s) + 3 us (s > 1),
// t_tile = 2 * 256 * TN * K / 3.9 TFLOP/s (one CU's measured rate), for
// tiles of 256 x TN.
void bf16_tail_plan(int64_t M, int64_t N, int64_t K, int cus, int TN, int &full, int &split,
                    int &tail) {
  const int64_t T = ((M + BM - 1) / BM) * ((N + TN - 1) / TN);
  const int64_t S = (K + BK - 1) / BK;
  full = (int)T;
  split = 1;
  tail = 0;
  const int64_t R = T % cus;
  if (R == 0) return;
  const double t_tile = 2.0 * BM * TN * (double)K / 3.9e6;          // us
  const double part_us = (double)BM * TN * 4 / 4.0e6;               // us per partial tile read
  double best = t_tile;
  int bs = 1;
  for (int s = 2; s <= 16 && S / s >= 4; ++s) {
    const double t = (double)((s * R + cus - 1) / cus) / s * t_tile + s * R * part_us + 3.0;
    if (t < best) {
      best = t;
      bs = s;
    }
  }
  if (bs == 1) return;
  full = (int)(T - R);
  split = bs;
  tail = (int)R;
}

}  // namespace

// tile width along N: 256 while both operands are under 4 GiB (the 32-bit
// row offsets of the 256 x 256 kernel), else 128
int bf16_tile_n(int64_t M, int64_t N, int64_t K) {
  const int64_t lim = (int64_t)1 << 32;
  return M * K * 2 < lim && N * K * 2 < lim ? t256::TBN : BN;
}

size_t bf16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  int full, split, tail;
  const int tn = bf16_tile_n(M, N, K);
  bf16_tail_plan(M, N, K, cu_count(), tn, full, split, tail);
  return (size_t)tail * split * BM * tn * sizeof(float);
}

hipError_t launch_bf16(const Bf16Args &p0, void *ws, hipStream_t stream) {
  if (p0.w_nvfp4) {
    const int tiles = ((p0.N + BN - 1) / BN) * ((p0.M + BM - 1) / BM);
    hipLaunchKernelGGL(bf16_gemm_kernel<true>, dim3(tiles), dim3(NTHR), 0, stream, p0);
    return hipGetLastError();
  }
  const int tn = bf16_tile_n(p0.M, p0.N, p0.K);
  const int tiles = ((p0.N + tn - 1) / tn) * ((p0.M + BM - 1) / BM);
  Bf16Args p = p0;
  int tail = 0;
  bf16_tail_plan(p.M, p.N, p.K, cu_count(), tn, p.full_tiles, p.split, tail);
  if (tail > 0 && ws == nullptr) {   // no workspace: whole tiles only
    p.full_tiles = tiles;
    p.split = 1;
    tail = 0;
  }
  p.part = (float *)ws;
  const dim3 grid(p.full_tiles + tail * p.split);
  if (tn == t256::TBN)
    hipLaunchKernelGGL(t256::bf16_gemm_256, grid, dim3(NTHR), 0, stream, p);
  else
    hipLaunchKernelGGL(bf16_gemm_kernel<false>, grid, dim3(NTHR), 0, stream, p);
  if (tail > 0) {
    if (tn == t256::TBN)
      hipLaunchKernelGGL(bf16_tail_sum<t256::TBN>, dim3(BM * t256::TBN / 2048, tail), dim3(256), 0,
                         stream, p);
    else
      hipLaunchKernelGGL(bf16_tail_sum<BN>, dim3(BM * BN / 2048, tail), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mg
