// gemm_w4a8.hip -- small-M (decode) TN GEMM of FP8 E4M3 per-token activations
// under NVFP4 weights on gfx950, through the exact E4M3 route of the
// metrale_circuit hardware::exec documentation (exec_of: NVFP4 weights under
// FP8 activations have no single-instruction MMA and take the exact route):
//
//   * weight codes -> E4M3 by the E2M1 -> E4M3 bit identity (value x 2^-6);
//   * one v_mfma_f32_32x32x16_fp8_fp8 per 16-element group, zero accumulator;
//   * acc = fma(64 * s_w[n,g], P_g, acc) in FP32 (the folded 2^6);
//   * epilogue: acc * a_tok[m] * S_w.
//
// The operation streams the weight (N*K/2 code bytes + N*K/16 scale bytes)
// once per 32 tokens, so it is arranged for HBM:
//   * HBM reads run fastest when a wave reads long contiguous runs of one
//     weight row, while the MFMA's B operand wants one weight row per lane.
//     A workgroup therefore loads its 128 weight rows x 256 K-elements
//     coalesced (8 lanes cover the 128-byte code run of one row), with the
//     rows' scale bytes and the token rows, into LDS; each wave then computes
//     its 32-row slab from LDS.  Code rows are XOR-swizzled in 16-byte chunks
//     so the 32 rows one operand read touches spread over the LDS banks;
//     token rows are padded by 8 bytes for the same reason.
//   * K is cut into 256-element ranges, two per workgroup (K = 14336 gives
//     28 splits and 1176 workgroups for N = 5376); both are requested at once
//     (register buffers), so the whole weight stream is in flight from the
//     start, and each range is staged and computed as soon as its own loads
//     land -- the work left after the last bytes arrive is one short range.
//   * the K ranges of a weight tile are split over ks workgroups (split-K);
//     each writes an FP32 partial, and a second kernel sums the partials in
//     split order 0..ks-1 -- results are bit-identical run to run.  (A split
//     that reduces in place needs its partials visible across the XCDs'
//     separate L2 caches within the kernel, which costs more than the second
//     launch.)
// Tokens sit on the MFMA's A side, padded to 32: lanes of token rows >= M
// read row 0 (those MFMA rows are never stored), and only the accumulator
// registers that hold real tokens are scaled.  Up to 64 tokens go through
// one launch as up to two 32-token blocks, each weight fragment converted
// once for both; more tokens take the tiled kernel (gemm_w4a8_tile.hip),
// where the per-group FMAs rather than the weight stream are the bound.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int NT = 128;       // weight rows per workgroup (4 waves x 32)
constexpr int KR = 256;       // K-elements per range
constexpr int RPW = 2;        // ranges per workgroup, all requested at once
constexpr int MS = 64;        // tokens per launch (up to 2 blocks of 32)
constexpr int TILE_M = 64;    // more tokens than this take the tiled kernel

constexpr int ROWB = KR / 2;          // code bytes per weight row per range
constexpr int CHUNKS = ROWB / 16;     // 16-byte chunks per code row (2 groups each)
constexpr int SB = KR / 16;           // scale bytes per row per range
constexpr int SROWF = SB + 2;         // LDS floats per scale row (padded: rows hit distinct banks)
constexpr int AROW = KR + 16;         // LDS bytes per token row (padded)

// MT token rows (8 per accumulator quad in use): 20992 bytes at MT = 8,
// 27520 at MT = 32
template <int MT>
struct Tile {
  static constexpr int AROWS = (MT * (KR / 16) + 255) / 256 * 256 / (KR / 16);  // rows the loads cover
  uint8_t w[NT * ROWB];
  float s[NT * SROWF];      // group scales decoded to FP32, times 64
  uint8_t a[AROWS * AROW];
};

constexpr int WCH = NT * CHUNKS / 256;          // code chunks per thread

// Code chunk c of weight row `row` (K-elements 32c .. 32c+31) sits at
// woff(row, c) with its four dwords reordered [d0 d2 d1 d3], where d0/d1 are
// the low/high halves of group 2c and d2/d3 those of group 2c+1: the lane
// that feeds MFMA K-half h then reads both groups' slices as one 8-byte word.
__device__ __forceinline__ int woff(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & (CHUNKS - 1))) << 4);
}

template <int MT>
struct RangeRegs {
  static constexpr int ACH = (MT * (KR / 16) + 255) / 256;  // token chunks per thread
  // global loads range_load issues per thread (its scale loads: one 8-byte
  // load when K % 256 == 0, else four 2-byte loads)
  template <bool SFAST>
  static constexpr int loads() { return WCH + (SFAST ? 1 : 4) + ACH; }
  u32x4 w[WCH];
  uint32_t s[4];   // scale bytes of row tid / 2, groups 8 (tid % 2) .. +7: two
                   // dwords (K % 256 == 0) or four 2-byte pairs, as loaded
  u32x4 a[ACH];
};

// Loads of K range [k0, k0 + klen) of this workgroup's weight tile and
// tokens.  Addresses are clamped in bounds and nothing is selected on the
// loaded data here -- a use of it would make the loads wait at once; the
// data past klen (or past the last token) is masked in range_store.
template <int MT, bool SFAST>
__device__ __forceinline__ void range_load(const W4A8Args &p, int n0, int k0, int klen, int tid,
                                           RangeRegs<MT> &r) {
  constexpr int ACH = RangeRegs<MT>::ACH;
  const int G = p.K / 16;
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + 256 * i, row = c / CHUNKS, ch = c % CHUNKS;
    const int n = n0 + row < p.N ? n0 + row : p.N - 1;
    const bool in = ch * 32 < klen;
    r.w[i] = *(const u32x4 *)(p.wq + (int64_t)n * (p.K / 2) + k0 / 2 + (in ? ch : 0) * 16);
  }
  {
    static_assert(SB == 16, "one scale row per thread pair");
    const int row = tid >> 1, q = tid & 1;
    const int n = n0 + row < p.N ? n0 + row : p.N - 1;
    const uint8_t *srow = p.ws + (int64_t)n * G + k0 / 16;
    if constexpr (SFAST) {  // K % 256 == 0: 8-byte aligned scale runs
      const bool in = 128 * q < klen;            // groups 8q.. of this range exist
      const u32x2 x = *(const u32x2 *)(srow + (in ? 8 * q : 0));
      r.s[0] = x[0];
      r.s[1] = x[1];
    } else {                // K % 32 == 0: 2-byte aligned, loaded in pairs
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 8 * q + 2 * e;             // within the range
        r.s[e] = *(const uint16_t *)(srow + (16 * g < klen ? g : 0));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + 256 * i, t = c / (KR / 16), ch = c % (KR / 16);
    const bool in = t < p.M && ch * 16 < klen;
    const int tt = t < p.M ? t : p.M - 1;
    r.a[i] = *(const u32x4 *)(p.aq + (int64_t)tt * p.K + k0 + (in ? ch : 0) * 16);
  }
}

template <int MT, bool SFAST>
__device__ __forceinline__ void range_store(Tile<MT> &tile, int M, int klen, int tid,
                                            const RangeRegs<MT> &r) {
  constexpr int ACH = RangeRegs<MT>::ACH;
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + 256 * i, row = c / CHUNKS, ch = c % CHUNKS;
    const u32x4 v = ch * 32 < klen ? r.w[i] : u32x4{0, 0, 0, 0};
    *(u32x4 *)(tile.w + woff(row, ch)) = u32x4{v[0], v[2], v[1], v[3]};
  }
  {
    const int row = tid >> 1, q = tid & 1;
    uint32_t sw[2];
    if constexpr (SFAST) {
      const bool in = 128 * q < klen;
      sw[0] = in ? r.s[0] : 0u;
      sw[1] = in ? r.s[1] : 0u;
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool in0 = 16 * (8 * q + 4 * e) < klen, in1 = 16 * (8 * q + 4 * e + 2) < klen;
        sw[e] = (in0 ? r.s[2 * e] : 0u) | ((in1 ? r.s[2 * e + 1] : 0u) << 16);
      }
    }
    float *dst = tile.s + row * SROWF + 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = sw[j >> 1] >> (16 * (j & 1));
      *(f32x2 *)(dst + 2 * j) = f32x2{e4m3_x64_to_f32_nan(w & 0xFFu), e4m3_x64_to_f32_nan((w >> 8) & 0xFFu)};
    }
  }
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    // (rows t >= M hold zeros; the tile has a row for every chunk loaded, so
    // the store needs no guard that a load could be sunk into)
    const int c = tid + 256 * i, t = c / (KR / 16), g = c % (KR / 16);
    // each 8-byte slice in even/odd byte order (the converted weight codes
    // come out in that order); the slices of groups 2c and 2c+1 that one
    // MFMA K-half reads are placed side by side: [lo(2c) lo(2c+1) | hi(2c) hi(2c+1)]
    const u32x4 av = t < M && 16 * g < klen ? r.a[i] : u32x4{0, 0, 0, 0};
    const uint64_t lo = e4m3x8_even_odd((uint64_t)av[0] | ((uint64_t)av[1] << 32));
    const uint64_t hi = e4m3x8_even_odd((uint64_t)av[2] | ((uint64_t)av[3] << 32));
    uint8_t *dst = tile.a + t * AROW + 32 * (g >> 1) + 8 * (g & 1);
    *(uint64_t *)dst = lo;
    *(uint64_t *)(dst + 16) = hi;
  }
}

// np pairs of 16-element groups (2 groups per code chunk) from the LDS tile
// QUADS = accumulator quads in use (8 tokens each); 0 means one token: only
// register 0 (token 0 in the lanes of K-half 0) is updated and stored.  Up to
// 4 quads fill one 32-token block; QUADS = 8 is 2 full blocks (64 tokens),
// each code fragment converted once for both.
template <int QUADS>
struct Acc {
  static constexpr int MT = QUADS == 0 ? 8 : 8 * QUADS;   // token rows in the LDS tile
  static constexpr int TB = QUADS <= 4 ? 1 : QUADS / 4;   // 32-token blocks
  static constexpr int NREG = QUADS == 0 ? 1 : (QUADS <= 4 ? 4 * QUADS : 16);  // registers in use per block
};

template <int QUADS, bool FULL>
__device__ __forceinline__ void compute_range(const Tile<Acc<QUADS>::MT> &tile, int row, int trow, int h, int np,
                                              f32x16 (&acc)[Acc<QUADS>::TB]) {
  constexpr int TB = Acc<QUADS>::TB;
  const uint8_t *wtile = tile.w + 8 * h;
  const uint8_t *arow = tile.a + trow * AROW + 16 * h;
  const float *srow = tile.s + row * SROWF;
  const f32x16 zero = {0};
  auto pair = [&](int c) {
    const uint64_t cw = *(const uint64_t *)(wtile + woff(row, c));
    const f32x2 sc = *(const f32x2 *)(srow + 2 * c);
    const float s0 = sc[0], s1 = sc[1];
    const uint64_t w0 = nvfp4x8_to_e4m3x8((uint32_t)cw), w1 = nvfp4x8_to_e4m3x8((uint32_t)(cw >> 32));
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const u32x4 av = *(const u32x4 *)(arow + 32 * AROW * b + 32 * c);
      const uint64_t a0 = (uint64_t)av[0] | ((uint64_t)av[1] << 32);
      const uint64_t a1 = (uint64_t)av[2] | ((uint64_t)av[3] << 32);
      const f32x16 p0 = mfma_fp8(a0, w0, zero);
      const f32x16 p1 = mfma_fp8(a1, w1, zero);
#pragma unroll
      for (int r = 0; r < Acc<QUADS>::NREG; ++r) acc[b][r] = __builtin_fmaf(s0, p0[r], acc[b][r]);
#pragma unroll
      for (int r = 0; r < Acc<QUADS>::NREG; ++r) acc[b][r] = __builtin_fmaf(s1, p1[r], acc[b][r]);
    }
  };
  if constexpr (FULL) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) pair(c);
  } else {
    for (int c = 0; c < np; ++c) pair(c);
  }
}

template <int QUADS>
__device__ __forceinline__ void compute_any(const Tile<Acc<QUADS>::MT> &tile, int row, int trow, int h, int klen,
                                            f32x16 (&acc)[Acc<QUADS>::TB]) {
  if (klen == KR)
    compute_range<QUADS, true>(tile, row, trow, h, CHUNKS, acc);
  else
    compute_range<QUADS, false>(tile, row, trow, h, klen / 32, acc);
}

// wait until at most `left` ranges' loads (LPR per range) are still in flight
template <int LPR>
__device__ __forceinline__ void wait_ranges_left(int left) {
  static_assert(RPW <= 4 && (RPW - 1) * LPR < 64, "vmcnt range");
  switch (left) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<LPR>(); break;
    case 2: wait_vmcnt<2 * LPR>(); break;
    default: wait_vmcnt<3 * LPR>(); break;
  }
}

// Workgroup id -> (weight tile, split).  A 128-byte line of a row's scale
// bytes covers SPL consecutive splits (SPL * RPW ranges of 16 scale bytes);
// the SPL workgroups that share those lines are given ids that are equal
// modulo 8, the number of XCDs that take workgroups round-robin, so they run
// on one XCD and the lines come from HBM once into its L2 rather than once
// per workgroup.  Ids that map past the last split return at once.
constexpr int XCDS = 8;
constexpr int SPL = 128 / (RPW * SB);
__device__ __forceinline__ bool split_of(int id, int tiles, int ks, int &nt, int &kc) {
  const int kq = (ks + SPL - 1) / SPL;                     // line groups per tile
  const int x = id % XCDS, slot = id / XCDS;
  const int lg = x + XCDS * (slot / SPL);
  if (lg >= tiles * kq) return false;
  nt = lg / kq;
  kc = (lg % kq) * SPL + slot % SPL;
  return kc < ks;
}

int split_grid(int tiles, int ks) {
  const int lgs = tiles * ((ks + SPL - 1) / SPL);
  return XCDS * SPL * ((lgs + XCDS - 1) / XCDS);
}

int splits(int64_t K) { return (int)(((K + KR - 1) / KR + RPW - 1) / RPW); }

template <int QUADS, bool SFAST>
__global__ __launch_bounds__(256) void w4a8_decode_kernel(W4A8Args p, int ks, float *part) {
  constexpr int MT = Acc<QUADS>::MT;
  __shared__ __attribute__((aligned(16))) Tile<MT> tile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  int nt, kc;
  if (!split_of(blockIdx.x, (p.N + NT - 1) / NT, ks, nt, kc)) return;
  const int n0 = nt * NT;
  const int nrange = (p.K + KR - 1) / KR;
  const int rbeg = kc * RPW;
  const int rend = rbeg + RPW < nrange ? rbeg + RPW : nrange;

  constexpr int TB = Acc<QUADS>::TB;
  const int row = wave * 32 + l32;
  // (with one block, token rows past M read row 0: never stored; with several
  // blocks every tile row exists and rows past M hold zeros)
  const int trow = TB > 1 || l32 < p.M ? l32 : 0;
  f32x16 acc[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) acc[b] = f32x16{0};

  // All of the workgroup's ranges (at most RPW) are requested at once into
  // register buffers, so the whole weight stream is in flight from the start;
  // each range is then staged through the one LDS tile and computed as soon as
  // its own loads have landed (loads complete in issue order, so range j waits
  // only for its batch), while the later ranges are still arriving.  A range
  // past the run is requested with length 0: its data is masked and only each
  // row's first chunk is touched.
  auto klen = [&](int rg) {
    return rg >= rend ? 0 : (p.K - rg * KR < KR ? p.K - rg * KR : KR);
  };
  auto kstart = [&](int rg) { return (rg < rend ? rg : rend - 1) * KR; };
  constexpr int LPR = RangeRegs<MT>::template loads<SFAST>();
  RangeRegs<MT> rr[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    range_load<MT, SFAST>(p, n0, kstart(rbeg + j), klen(rbeg + j), tid, rr[j]);
    __builtin_amdgcn_sched_barrier(0);  // ranges are issued in order
  }
  // (Every range, even an empty one, is stored and computed with no branch
  // around it: a load whose only use sits in a branch is moved into it, and
  // the waits before it then cover every load in flight.)
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    if (j > 0) {  // every wave is done reading the previous range
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
    wait_ranges_left<LPR>(RPW - 1 - j);
    range_store<MT, SFAST>(tile, p.M, klen(rbeg + j), tid, rr[j]);
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    compute_any<QUADS>(tile, row, trow, h, klen(rbeg + j), acc);
  }

  const int n = n0 + row;
  if (ks == 1) {
    if (n >= p.N) return;
    const float sw = *p.Sw;
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int r = 0; r < Acc<QUADS>::NREG; ++r) {
        const int t = 32 * b + acc_row(r, lane);
        if (t >= p.M) continue;
        const float v = acc[b][r] * (p.atok[t] * sw);
        if (p.out_f32)
          ((float *)p.C)[(int64_t)t * p.N + n] = v;
        else
          ((uint16_t *)p.C)[(int64_t)t * p.N + n] = (uint16_t)f32_to_bf16_rne(v);
      }
    return;
  }

  if (n < p.N) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int r = 0; r < Acc<QUADS>::NREG; ++r) {
        const int t = 32 * b + acc_row(r, lane);
        if (t < p.M) part[((int64_t)kc * p.M + t) * p.N + n] = acc[b][r];
      }
  }
}

// C[t,n] = (sum over splits s = 0..ks-1, in order, of part[s,t,n]) * a_tok[t] * S_w.
// One element per thread.  The scales and the first CH partials are all
// requested up front (addresses past ks repeat the last split and are not
// added), so a decode-sized reduction waits on one memory latency.
__global__ __launch_bounds__(64) void w4a8_splitk_reduce(W4A8Args p, int ks, const float *part) {
  constexpr int CH = 32;
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  const int64_t mn = (int64_t)p.M * p.N;
  if (i >= mn) return;
  const int t = mn <= 0x7FFFFFFF ? (int)((uint32_t)i / (uint32_t)p.N) : (int)(i / p.N);
  const float scale = p.atok[t] * *p.Sw;
  float x[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) x[j] = part[(int64_t)(j < ks ? j : ks - 1) * mn + i];
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < CH; ++j) v = j < ks ? v + x[j] : v;
  for (int s = CH; s < ks; ++s) v += part[(int64_t)s * mn + i];   // ks > CH: K > 16384
  v *= scale;
  if (p.out_f32)
    ((float *)p.C)[i] = v;
  else
    ((uint16_t *)p.C)[i] = (uint16_t)f32_to_bf16_rne(v);
}

template <int QUADS>
void launch_one(const W4A8Args &p, int ks, float *part, hipStream_t stream) {
  const dim3 grid(split_grid((p.N + NT - 1) / NT, ks));
  if (p.K % 256 == 0)
    hipLaunchKernelGGL((w4a8_decode_kernel<QUADS, true>), grid, dim3(256), 0, stream, p, ks, part);
  else
    hipLaunchKernelGGL((w4a8_decode_kernel<QUADS, false>), grid, dim3(256), 0, stream, p, ks, part);
}

}  // namespace

size_t w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  int ks = splits(K);
  if (M > TILE_M) {             // the tiled kernel
    int gpw;
    w4a8_tile_split(M, N, K, ks, gpw);
  }
  return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int64_t w4a8_max_n() { return (int64_t)1 << 30; }

hipError_t launch_w4a8(const W4A8Args &p0, hipStream_t stream) {
  if (p0.M > TILE_M) {
    int ks, gpw;
    w4a8_tile_split(p0.M, p0.N, p0.K, ks, gpw);
    float *part = ks > 1 ? (float *)p0.work : nullptr;
    hipError_t e = launch_w4a8_tile(p0, ks, gpw, part, stream);
    if (e != hipSuccess || ks == 1) return e;
    const int64_t mn = (int64_t)p0.M * p0.N;
    hipLaunchKernelGGL(w4a8_splitk_reduce, dim3((unsigned)((mn + 63) / 64)), dim3(64), 0, stream, p0,
                       ks, part);
    return hipGetLastError();
  }
  const int ks = splits(p0.K);
  float *part = ks > 1 ? (float *)p0.work : nullptr;
  for (int m0 = 0; m0 < p0.M; m0 += MS) {
    W4A8Args p = p0;
    p.M = p0.M - m0 < MS ? p0.M - m0 : MS;
    p.aq = p0.aq + (int64_t)m0 * p0.K;
    p.atok = p0.atok + m0;
    p.C = (char *)p0.C + (int64_t)m0 * p0.N * (p0.out_f32 ? 4 : 2);
    if (p.M > 32) launch_one<8>(p, ks, part, stream);
    else if (p.M > 24) launch_one<4>(p, ks, part, stream);
    else if (p.M > 16) launch_one<3>(p, ks, part, stream);
    else if (p.M > 8) launch_one<2>(p, ks, part, stream);
    else if (p.M > 1) launch_one<1>(p, ks, part, stream);
    else launch_one<0>(p, ks, part, stream);
    if (ks > 1) {
      const int64_t mn = (int64_t)p.M * p.N;
      hipLaunchKernelGGL(w4a8_splitk_reduce, dim3((unsigned)((mn + 63) / 64)), dim3(64), 0,
                         stream, p, ks, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mg
