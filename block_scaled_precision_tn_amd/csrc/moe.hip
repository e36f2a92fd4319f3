// moe.hip -- MXFP8 grouped mixture-of-experts GLU on gfx950 (the MXFP8 x
// MXFP8 -> BF16 MoE GLU of the FlashInfer swapab_cutedsl_megakernel skill
// page, Layout section; that page names a generic MXFP8 GLU reference whose
// computation this restates):
//
//   for every token t and routing slot j with expert e = ids[t,j]:
//     [g ; u] = x_t . w13[e]^T   (K = H; rows [0,I) gate, [I,2I) up)
//     h = silu(g) * u            (FP32)
//     h -> MXFP8 (E8M0 per 32 along I; OCP MX rule, E4M3 saturating)
//     y = h . w2[e]^T            (K = I)
//     out[t] += ids weight * y   (FP32), then BF16
//
// Stream-ordered kernels:
//   k_prep   zero the expert counters
//   k_count  per-expert histogram; each entry's rank within its expert
//   k_scan   expert row offsets and the tile list (128 or 256 rows per
//            tile; the grouped GEMM grids need no host sync)
//   k_scatter each entry's sorted row (entries grouped by expert)
//   k_gateup grouped GEMM on the E8M0-scaled FP8 MFMA with gathered token
//            rows; epilogue: GLU, MXFP8 re-quantisation of h (block amax by
//            cross-lane max), h stored in expert-sorted order
//   k_down   grouped GEMM of sorted h rows against w2[e]; epilogue: times the
//            routing weight, stored FP32 per routed row (expert-sorted order)
//   k_combine out[t] = sum over slots j = 0..topk-1, in order, of the stored
//            rows of (t, j), then BF16 (deterministic: no atomics)
#include "common.h"
#include "kernels.h"
#include "quant.h"

namespace mg {
namespace {

constexpr int BM = 128;       // rows (routing entries) per tile
constexpr int BNI = 64;       // intermediate columns per gate/up tile (x2 rows of w13)
constexpr int BNH = 128;      // hidden columns per down tile
constexpr int BK = 64;        // K per LDS stage (two 32-element scale blocks)
constexpr int CSTRIDE = 32;   // uint32s between two experts' row counters

struct Layout {
  size_t counts, offs, meta, sorted, pos, wsorted, tile_e, tile_r, tile_n, hq, hs, y, total;
  int R, maxtiles;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// fp4: h stored as NVFP4 (I/2 code bytes, I/16 scale bytes per row) rather
// than MXFP8 (I, I/32)
Layout layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk, bool fp4 = false) {
  Layout L;
  L.R = (int)(T * topk);
  L.maxtiles = (int)((L.R + BM - 1) / BM + E);
  size_t o = 0;
  L.counts = o; o += up256(sizeof(uint32_t) * CSTRIDE * (size_t)E);   // one 128-byte line each
  L.offs = o;   o += up256(sizeof(int32_t) * (size_t)E);
  L.meta = o;   o += up256(sizeof(int32_t) * 4);                 // [0] = number of tiles
  L.sorted = o; o += up256(sizeof(int32_t) * (size_t)L.R);
  L.pos = o;    o += up256(sizeof(int32_t) * (size_t)L.R);          // sorted row of each entry
  L.wsorted = o; o += up256(sizeof(float) * (size_t)L.R);           // routing weight of each sorted row
  L.tile_e = o; o += up256(sizeof(int32_t) * (size_t)L.maxtiles);
  L.tile_r = o; o += up256(sizeof(int32_t) * (size_t)L.maxtiles);
  L.tile_n = o; o += up256(sizeof(int32_t) * (size_t)L.maxtiles);
  L.hq = o;     o += up256((size_t)L.R * (size_t)(fp4 ? I / 2 : I));
  L.hs = o;     o += up256((size_t)L.R * (size_t)(fp4 ? I / 16 : I / 32));
  L.y = o;      o += up256(sizeof(float) * (size_t)L.R * (size_t)H);  // weighted down rows
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- routing
// Expert e's row counter is counts[CSTRIDE * e]: one 128-byte line per
// expert, so the workgroups' atomic reservations on different experts go to
// different lines (and L2 channels) instead of queueing on two lines.
__global__ void k_prep(uint32_t *counts, int E) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) counts[CSTRIDE * i] = 0u;
}

// rank of each entry within its expert (arrival order); out-of-range ids are
// dropped.  Row order within an expert does not change any result: every
// row's GEMMs and re-quantisation are independent of the other rows.
__global__ __launch_bounds__(1024) void k_count(const int32_t *ids, int R, int E,
                                                uint32_t *counts, int32_t *rank) {
  // ranks within the workgroup from LDS counters, then one global atomic per
  // (workgroup, expert) reserves the workgroup's run of ranks
  __shared__ uint32_t s_cnt[1024], s_base[1024];
  const int tid = threadIdx.x, i = blockIdx.x * 1024 + tid;
  if (tid < E) s_cnt[tid] = 0u;
  __syncthreads();
  const int e = i < R ? ids[i] : -1;
  const bool ok = e >= 0 && e < E;
  const uint32_t lr = ok ? atomicAdd(&s_cnt[e], 1u) : 0u;
  __syncthreads();
  if (tid < E && s_cnt[tid] != 0u) s_base[tid] = atomicAdd(&counts[CSTRIDE * tid], s_cnt[tid]);
  __syncthreads();
  if (i < R) rank[i] = ok ? (int32_t)(s_base[e] + lr) : -1;
}

// one workgroup: exclusive scans of the expert counts (row offsets) and of
// their tile counts (tile list: expert, first row, rows)
template <int TM>
__global__ __launch_bounds__(256) void k_scan(const uint32_t *counts, int E, int32_t *offs,
                                              int32_t *meta, int32_t *tile_e, int32_t *tile_r,
                                              int32_t *tile_n) {
  __shared__ int s_rows[256], s_tiles[256];
  const int tid = threadIdx.x;
  constexpr int PER = 4;                       // experts per thread (E <= 1024)
  int rows[PER], tiles[PER], r = 0, t = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid * PER + k;
    const int c = e < E ? (int)counts[CSTRIDE * e] : 0;
    rows[k] = c;
    tiles[k] = (c + TM - 1) / TM;
    r += c;
    t += tiles[k];
  }
  s_rows[tid] = r;
  s_tiles[tid] = t;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {          // inclusive scan over threads
    const int ar = tid >= o ? s_rows[tid - o] : 0, at = tid >= o ? s_tiles[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += ar;
    s_tiles[tid] += at;
    __syncthreads();
  }
  int rb = s_rows[tid] - r, tb = s_tiles[tid] - t;
  if (tid == 255) meta[0] = s_tiles[255];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid * PER + k;
    if (e < E) {
      offs[e] = rb;
      for (int q = 0; q < tiles[k]; ++q) {
        tile_e[tb + q] = e;
        tile_r[tb + q] = rb + q * TM;
        tile_n[tb + q] = rows[k] - q * TM < TM ? rows[k] - q * TM : TM;
      }
    }
    rb += rows[k];
    tb += tiles[k];
  }
}

// sorted row of each entry, and the entry and routing weight of each sorted row
__global__ void k_scatter(const int32_t *ids, const float *tw, int R, const int32_t *offs,
                          int32_t *pos, int32_t *sorted, float *wsorted) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < R) {
    const int rk = pos[i];                     // rank from k_count, or -1
    if (rk >= 0) {
      const int p = offs[ids[i]] + rk;
      pos[i] = p;
      sorted[p] = i;
      wsorted[p] = tw[i];
    }
  }
}

// ------------------------------------------------------- MX GEMM mainloop
// A: 128 rows, B: 128 rows, both MXFP8 with K = Ktot (a multiple of 64).
// Wave (wm, wn) computes rows wm*64 + [0,64) against the two 32-row B slabs
// bsel[0], bsel[1]; acc[i][j] is the 32x32 block (A slab i, B slab j).
//
// Operands go from global memory straight into LDS (global_load_lds: lane i
// of an instruction lands at its LDS base + i * size), three stages of 64 K
// deep, so two stages are in flight while one is computed.  Per stage and
// operand a 128 x 64-byte code tile, rows XOR-swizzled in 16-byte chunks (see
// mx_off) so MFMA fragment reads hit distinct banks; the rows' E8M0 scale
// bytes (A rows, then B rows) arrive 8 stages at a time when K % 512 == 0,
// else per stage (see mx_issue_sc16 / mx_issue_sc2).  A rows are gathered:
// every lane holds the global row pointers of the rows it loads.

constexpr int MX_CODE = BM * BK;          // bytes of one operand's codes per stage
constexpr int SCH = 8;                    // stages per scale chunk (K % 512 == 0)
constexpr int MX_SCC = 2 * BM * 2 * SCH;  // scale bytes per chunk: 16 per row (A rows then B rows)
constexpr int MX_SCS = 2 * BM * 4;        // scale bytes per stage otherwise: one dword per row

// chunk `chunk` (16 bytes) of 64-byte row `row`: XOR-ed with (row / 4) % 4,
// so 16 consecutive rows at one chunk index cover all 64 LDS banks
__device__ __forceinline__ int mx_off(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 2) & 3)) << 4);
}

struct MxRows {
  const uint8_t *a[2], *b[2];   // code rows this lane loads: rows 16 (2 wave + j) + lane / 4
  const uint8_t *s;             // scale row of row (64 wave + lane) % 128 (A if < 128, else B)
};

// lane's loads of one stage at k0: 2 A + 2 B code chunks
__device__ __forceinline__ void mx_issue(const MxRows &r, int k0, uint8_t *la, uint8_t *lb, int wave,
                                         int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = 2 * wave + j, row = 16 * blk + (lane >> 2), slot = lane & 3;
    const int chunk = slot ^ ((row >> 2) & 3);
    dma16(r.a[j] + k0 + 16 * chunk, la + 1024 * blk);
    dma16(r.b[j] + k0 + 16 * chunk, lb + 1024 * blk);
  }
}

// Scale bytes.  When the scale rows are a multiple of 16 bytes long (K % 512
// == 0), a lane loads its row's 16 bytes for 8 stages at once (chunk c:
// stages 8c .. 8c+7) into registers and stores them a stage later to
// ls + 16 * (64 wave + lane) (a plain store: a direct-to-LDS load into a
// buffer chosen at run time would make every later LDS read wait for all
// loads in flight); otherwise it loads the 2 bytes of one stage directly into
// one dword per lane (low half) at ls + 4 * (64 wave + lane).  Each such
// load touches one row per lane, and the texture path's cost grows with the
// rows an instruction touches.
__device__ __forceinline__ u32x4 mx_load_sc16(const MxRows &r, int c) {
  return *(const u32x4 *)(r.s + 16 * c);
}
__device__ __forceinline__ void mx_issue_sc2(const MxRows &r, int k0, uint8_t *ls, int wave) {
  dma2(r.s + k0 / 32, ls + 256 * wave);
}

// A stage's MFMAs from one LDS slot: fragments of the wave's two A slabs and
// NB B slabs, and their scales at ls + rs * row (A) / ls + rs * (BM + row) (B).
template <int NB>
__device__ __forceinline__ void mx_stage(const uint8_t *la, const uint8_t *lb, const uint8_t *ls, int rs,
                                         const int bsel[NB], int wm, int h, int l32,
                                         f32x16 (&acc)[2][NB]) {
  i32x8 fa[2], fb[NB];
  int sa[2], sb[NB];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wm * 64 + i * 32 + l32;
    const u32x4 lo = *(const u32x4 *)(la + mx_off(row, h));
    const u32x4 hi = *(const u32x4 *)(la + mx_off(row, 2 + h));
    fa[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sa[i] = ls[rs * row];
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int row = bsel[j] + l32;
    const u32x4 lo = *(const u32x4 *)(lb + mx_off(row, h));
    const u32x4 hi = *(const u32x4 *)(lb + mx_off(row, 2 + h));
    fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sb[j] = ls[rs * (BM + row)];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = mfma_mx_fp8(fa[i], fb[j], acc[i][j], sa[i], sb[j]);
}

// Per-stage scale loads (any K % 64 == 0): a three-slot ring of code and
// scale slots, each a separate array so the compiler can tell loads landing
// in one slot from reads of another; stage s+2 is loaded while stage s is
// computed.
template <int NB>
__device__ __forceinline__ void mx_mainloop_sc2(const MxRows &rows, int Ktot, const int bsel[NB],
                                                f32x16 (&acc)[2][NB]) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[MX_CODE], a1[MX_CODE], a2[MX_CODE];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[MX_CODE], b1[MX_CODE], b2[MX_CODE];
  __shared__ __attribute__((aligned(1024))) uint8_t c0[MX_SCS], c1[MX_SCS], c2[MX_SCS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, h = lane >> 5, l32 = lane & 31;
  const int S = Ktot / BK;
  constexpr int LOADS = 5;   // direct loads per lane per stage: 4 code chunks, 1 scale pair

  auto step = [&](int s, const uint8_t *la, const uint8_t *lb, const uint8_t *lc, uint8_t *na,
                  uint8_t *nb, uint8_t *nc) {
    __builtin_amdgcn_sched_barrier(0);
    // stage s has landed once at most stage s+1's loads are outstanding; the
    // bare s_barrier (a fenced one would wait for every load in flight)
    wait_vmcnt<LOADS>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // stage s+2 into the slot stage s-1 used (every wave is past it); stages
    // past the end reload the last one (never computed)
    const int t = s + 2 < S ? s + 2 : S - 1;
    mx_issue_sc2(rows, t * BK, nc, wave);
    mx_issue(rows, t * BK, na, nb, wave, lane);
    mx_stage<NB>(la, lb, lc + h, 4, bsel, wm, h, l32, acc);
  };
  mx_issue_sc2(rows, 0, c0, wave);
  mx_issue(rows, 0, a0, b0, wave, lane);
  mx_issue_sc2(rows, (1 < S ? 1 : 0) * BK, c1, wave);
  mx_issue(rows, (1 < S ? 1 : 0) * BK, a1, b1, wave, lane);
  // whole ring turns, then the last one or two stages: the loop has a single
  // exit, which keeps each accumulator in one set of registers
  const int full = S - S % 3;
  for (int s = 0; s < full; s += 3) {
    step(s, a0, b0, c0, a2, b2, c2);
    step(s + 1, a1, b1, c1, a0, b0, c0);
    step(s + 2, a2, b2, c2, a1, b1, c1);
  }
  if (S % 3 >= 1) step(full, a0, b0, c0, a2, b2, c2);
  if (S % 3 == 2) step(full + 1, a1, b1, c1, a0, b0, c0);
  wait_vmcnt<0>();
  // the slots are reused by the next tile only after this barrier
  __builtin_amdgcn_s_barrier();
}

// Scale chunks (K % 512 == 0): a four-slot code ring, stage s+3 loaded while
// stage s is computed, and the loop walks one scale chunk (8 stages, two
// ring turns) per iteration, so every slot is fixed at compile time.  Each
// lane loads its row's 16 scale bytes of chunk c+1 into registers at the
// start of chunk c and stores them (a plain LDS store) into the chunk buffer
// not in use at its last stage; every read of a scale buffer then has a
// known object that no direct-to-LDS load writes.
template <int NB>
__device__ __forceinline__ void mx_mainloop_sc16(const MxRows &rows, int Ktot, const int bsel[NB],
                                                 f32x16 (&acc)[2][NB]) {
  // (one array per slot, A codes then B codes: the compiler tracks only a
  // few distinct targets of direct-to-LDS loads before it makes every LDS
  // read wait for all of them)
  __shared__ __attribute__((aligned(1024))) uint8_t q0[2 * MX_CODE], q1[2 * MX_CODE], q2[2 * MX_CODE],
      q3[2 * MX_CODE];
  __shared__ __attribute__((aligned(1024))) uint8_t cs[2][MX_SCC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, h = lane >> 5, l32 = lane & 31;
  const int S = Ktot / BK, nch = S / SCH;
  // stage s has landed once at most the code loads of stages s+1 and s+2
  // (4 each) are outstanding, plus, for the first three stages of a chunk,
  // the next chunk's scale load (issued after their code loads)

  uint8_t *const la[4] = {q0, q1, q2, q3};
  uint8_t *const lb[4] = {q0 + MX_CODE, q1 + MX_CODE, q2 + MX_CODE, q3 + MX_CODE};
  u32x4 scr = mx_load_sc16(rows, 0);
  mx_issue(rows, 0, la[0], lb[0], wave, lane);
  mx_issue(rows, (1 < S ? 1 : 0) * BK, la[1], lb[1], wave, lane);
  mx_issue(rows, (2 < S ? 2 : S - 1) * BK, la[2], lb[2], wave, lane);
  *(u32x4 *)(cs[0] + 16 * tid) = scr;   // ordered before the first reads by the first barrier
  for (int c = 0; c < nch; ++c) {
    scr = mx_load_sc16(rows, c + 1 < nch ? c + 1 : c);
    const uint8_t *lsc = cs[c & 1] + h;
#pragma unroll
    for (int j = 0; j < SCH; ++j) {
      const int s = SCH * c + j;
      __builtin_amdgcn_sched_barrier(0);
      if (j < 3)
        wait_vmcnt<9>();
      else
        wait_vmcnt<8>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // stage s+3 into the slot stage s-1 used (every wave is past it);
      // stages past the end reload the last one (never computed)
      mx_issue(rows, (s + 3 < S ? s + 3 : S - 1) * BK, la[(j + 3) & 3], lb[(j + 3) & 3], wave, lane);
      if (j == SCH - 1) *(u32x4 *)(cs[(c + 1) & 1] + 16 * tid) = scr;
      mx_stage<NB>(la[j & 3], lb[j & 3], lsc + 2 * j, 16, bsel, wm, h, l32, acc);
    }
  }
  wait_vmcnt<0>();
  // the slots are reused by the next tile only after this barrier
  __builtin_amdgcn_s_barrier();
}

template <int NB, bool SC16>
__device__ __forceinline__ void mx_mainloop(const MxRows &rows, int Ktot, const int bsel[NB],
                                            f32x16 (&acc)[2][NB]) {
  if constexpr (SC16)
    mx_mainloop_sc16<NB>(rows, Ktot, bsel, acc);
  else
    mx_mainloop_sc2<NB>(rows, Ktot, bsel, acc);
}

// max over the 32 lanes that share (lane / 32): within each row of 16 lanes
// by DPP on the vector ALU (the other lane of the pair, of the quad's pair,
// the mirror lane of the half row, of the row), then one lane exchange with
// the other row of the 32
__device__ __forceinline__ float dpp_max(float v, int ctrl_kind) {
  int o;
  switch (ctrl_kind) {
    case 0: o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return fmaxf(v, __builtin_bit_cast(float, o));
}
__device__ __forceinline__ float row_max16(float v) {
  v = dpp_max(v, 0);
  v = dpp_max(v, 1);
  v = dpp_max(v, 2);
  return dpp_max(v, 3);
}
__device__ __forceinline__ float max32_lanes(float v) {
  v = row_max16(v);
  return fmaxf(v, __shfl_xor(v, 16, 64));
}

template <bool SC16>
__global__ __launch_bounds__(256) void k_gateup(MoeArgs p, const int32_t *meta,
                                                const int32_t *sorted, const int32_t *tile_e,
                                                const int32_t *tile_r, const int32_t *tile_n,
                                                uint8_t *hq, uint8_t *hs) {
  const int tile = blockIdx.y;
  if (tile >= meta[0]) return;
  const int e = tile_e[tile], r0 = tile_r[tile], nrows = tile_n[tile];
  const int i0 = blockIdx.x * BNI;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31;
  const int H = p.H, I = p.I;

  // A rows: gathered token rows (rows past the tile read the first entry's
  // token: never stored); B rows 0..63: gate i0+row, 64..127: up I+i0+row-64
  auto arow = [&](int row) {
    const int t = sorted[r0 + (row < nrows ? row : 0)] / p.topk;
    return p.xq + (int64_t)t * H;
  };
  auto brow = [&](int row) { return row < BNI ? i0 + row : I + i0 + (row - BNI); };
  MxRows rows;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    rows.a[j] = arow(row);
    rows.b[j] = p.w13q + ((int64_t)e * 2 * I + brow(row)) * H;
  }
  {
    const int q = 64 * wave + lane, row = q & 127;
    if (q < 128) {
      const int t = sorted[r0 + (row < nrows ? row : 0)] / p.topk;
      rows.s = p.xs + (int64_t)t * (H / 32);
    } else {
      rows.s = p.w13s + ((int64_t)e * 2 * I + brow(row)) * (H / 32);
    }
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{0};
  const int bsel[2] = {wn * 32, BNI + wn * 32};  // gate slab, up slab of the same columns
  mx_mainloop<2, SC16>(rows, H, bsel, acc);

  // epilogue: h = silu(g) * u, MXFP8 block of 32 columns = this wave's 32 lanes
  const int col = i0 + wn * 32 + l32;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + acc_row(r, lane);
      const float g = acc[i][0][r], u = acc[i][1][r];
      const float hv = (g / (1.0f + expf(-g))) * u;
      const float amax = max32_lanes(fabsf(hv));
      uint32_t sbyte, code;
      if (amax == 0.0f) {
        sbyte = 0u;
        code = 0u;
      } else {
        int X = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF) - 127 - 8;
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
        sbyte = (uint32_t)(X + 127);
        code = f32_to_e4m3_rne_sat(__builtin_ldexpf(hv, -X));
      }
      if (row < nrows) {
        const int64_t srow = r0 + row;
        if (p.dbg_gu) {
          float *d = p.dbg_gu + (int64_t)sorted[srow] * (2 * I);
          d[col] = g;
          d[I + col] = u;
        }
        hq[srow * I + col] = (uint8_t)code;
        if (l32 == 0) hs[srow * (I / 32) + col / 32] = (uint8_t)sbyte;
        if (p.dbg_h) {
          const int64_t ent = sorted[srow];
          uint8_t *d = p.dbg_h + ent * (int64_t)(I + I / 32);
          d[col] = (uint8_t)code;
          if (l32 == 0) d[I + col / 32] = (uint8_t)sbyte;
        }
      }
    }
}

template <bool SC16>
__global__ __launch_bounds__(256) void k_down(MoeArgs p, const int32_t *meta, const float *wsorted,
                                              const int32_t *tile_e, const int32_t *tile_r,
                                              const int32_t *tile_n, const uint8_t *hq,
                                              const uint8_t *hs, float *y) {
  __shared__ float s_w[256];   // routing weight of tile row t at s_w[t] (and s_w[128 + t])
  const int tile = blockIdx.y;
  if (tile >= meta[0]) return;
  const int e = tile_e[tile], r0 = tile_r[tile], nrows = tile_n[tile];
  const int n0 = blockIdx.x * BNH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31;
  const int H = p.H, I = p.I;
  // the tile rows' routing weights, requested before the main loop's loads
  // (so they have landed long before the epilogue needs them)
  const float wrow = wsorted[r0 + ((tid & 127) < nrows ? (tid & 127) : 0)];

  // A rows: sorted h rows (rows past the tile read its first row: never
  // stored); B rows: w2[e] rows n0 + row (past H: the last row, never stored)
  MxRows rows;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * (2 * wave + j) + (lane >> 2);
    rows.a[j] = hq + (int64_t)(r0 + (row < nrows ? row : 0)) * I;
    rows.b[j] = p.w2q + ((int64_t)e * H + (n0 + row < H ? n0 + row : H - 1)) * I;
  }
  {
    const int q = 64 * wave + lane, row = q & 127;
    if (q < 128)
      rows.s = hs + (int64_t)(r0 + (row < nrows ? row : 0)) * (I / 32);
    else
      rows.s = p.w2s + ((int64_t)e * H + (n0 + row < H ? n0 + row : H - 1)) * (I / 32);
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{0};
  const int bsel[2] = {wn * 64, wn * 64 + 32};
  mx_mainloop<2, SC16>(rows, I, bsel, acc);
  s_w[tid] = wrow;
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + acc_row(r, lane);
      if (row >= nrows) continue;
      const float w = s_w[row];
      float *yrow = y + (int64_t)(r0 + row) * H;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
        if (n < H) yrow[n] = acc[i][j][r] * w;
      }
    }
}

// ----------------------------------- grouped GEMMs on 256 x 256 tiles
// For the large calls (H and I multiples of 512) both grouped GEMMs run on
// 256-row tiles of routed rows (the tile list is built for 256 rows) against
// 256 weight rows: gate/up takes 128 gate and the 128 matching up rows (128
// h columns), down 256 hidden columns.  Eight waves (4 x 2) each compute
// 64 x 128 (2 x 4 blocks of 32 x 32 on the E8M0-scaled 32x32x64 FP8 MFMA),
// so a wave reads 6 operand fragments per 8 MFMAs (a 64 x 64 wave tile
// reads 4 per 4).  K is staged 128 bytes per row (8 rows x 128 bytes per
// load instruction: whole cache lines) through two 64 KiB LDS slots: stage
// s+2 is requested right after the barrier that follows the last read of
// stage s.  Rows are XOR-swizzled in 16-byte chunks as in the BF16 kernel.
// A lane's row offsets are fixed for the tile (gathered rows included) and
// stay in registers; only the operand base moves along K.  Each row's E8M0
// scale bytes arrive 16 at a time (four stages) straight into a
// double-buffered LDS chunk.  Within a K-step the B fragments are read one
// block column ahead of the MFMAs that use them.  A wave whose 64 rows all
// lie past the tile's routed rows skips its MFMAs.
namespace t2 {

constexpr int TM = 256, TN = 256, TK = 128;   // routed rows, weight rows, K bytes per stage
constexpr int NT = 512;
constexpr int STG = TM * TK;                  // bytes of one operand's codes per stage
constexpr int CHK = 4;                        // stages per scale chunk (16 bytes per row)

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * TK + ((chunk ^ ((row >> 1) & 7)) << 4);
}
// lane's j-th load of a stage (j < 4): row 8 (4 wave + j) + lane / 8, its
// LDS slot lane % 8 holds global chunk slot ^ ((row / 2) % 8)
__device__ __forceinline__ int ld_row(int wave, int j, int lane) { return 8 * (4 * wave + j) + (lane >> 3); }
__device__ __forceinline__ int ld_chunk(int row, int lane) { return (lane & 7) ^ ((row >> 1) & 7); }

__device__ __forceinline__ void issue(const uint8_t *base, int k0, const uint32_t (&off)[4],
                                      uint32_t lds, int wave) {
  const uint8_t *b = base + k0;
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16_s(off[j], b, lds + 1024u * (4 * wave + j));
}

template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}

template <bool GU>
__global__ __launch_bounds__(NT, 1) void k_mx256(MoeArgs p, const int32_t *meta,
                                                 const int32_t *sorted, const float *wsorted,
                                                 const int32_t *tile_e, const int32_t *tile_r,
                                                 const int32_t *tile_n, uint8_t *hq, uint8_t *hs,
                                                 float *y) {
  __shared__ __attribute__((aligned(1024))) uint8_t la0[STG], la1[STG], lb0[STG], lb1[STG];
  __shared__ __attribute__((aligned(16))) uint8_t scs[2][2 * TM * 16];   // [chunk & 1][row][16]
  __shared__ float s_w[TM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int H = p.H, I = p.I;
  const int K = GU ? H : I;
  // One workgroup per CU, each walking a list of (tile, column block)
  // items: workgroup w runs on XCD w % 8, and XCD x takes the x-th eighth
  // of the expert-ordered tile list, all column blocks of a tile next to
  // each other.  The 32 workgroups of an XCD then work on the same few row
  // tiles (which share gathered rows) of the same few experts (whose row
  // tiles share each weight slab) at once, from that XCD's L2.
  const int ncol = GU ? I / (TN / 2) : (H + TN - 1) / TN;
  const int nT = meta[0];
  const int xcd = blockIdx.x % 8, nslot = ((int)gridDim.x - xcd + 7) / 8;
  const int lo = (int)((int64_t)nT * xcd / 8), hi = (int)((int64_t)nT * (xcd + 1) / 8);
  const int items = (hi - lo) * ncol;
  for (int item = blockIdx.x / 8; item < items; item += nslot) {
  const int tile = lo + item / ncol;
  const int e = tile_e[tile], r0 = tile_r[tile], nrows = tile_n[tile];
  const int c0 = (item % ncol) * (GU ? TN / 2 : TN);   // first h column / hidden column

  // A: gathered token rows (gate/up) or sorted h rows (down); rows past the
  // tile read its first row (never stored).  B: gate rows c0.., then up rows
  // I + c0.. (gate/up), or w2 rows c0.. clamped to H (down).
  const uint8_t *abase = GU ? p.xq : hq;
  const uint8_t *bbase = GU ? p.w13q + (int64_t)e * 2 * I * H : p.w2q + (int64_t)e * H * I;
  auto a_row = [&](int row) -> int {
    const int rr = row < nrows ? row : 0;
    return GU ? sorted[r0 + rr] / p.topk : r0 + rr;
  };
  auto b_row = [&](int row) -> int {
    if (GU) return row < TN / 2 ? c0 + row : I + c0 + (row - TN / 2);
    return c0 + row < H ? c0 + row : H - 1;
  };
  uint32_t offa[4], offb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = ld_row(wave, j, lane), ch = ld_chunk(row, lane);
    offa[j] = (uint32_t)a_row(row) * (uint32_t)K + 16u * ch;
    offb[j] = (uint32_t)b_row(row) * (uint32_t)K + 16u * ch;
  }
  // this thread's scale row: A row tid (< 256) or B row tid - 256
  const uint8_t *srow;
  if (tid < TM)
    srow = (GU ? p.xs : hs) + (int64_t)a_row(tid) * (K / 32);
  else
    srow = (GU ? p.w13s + (int64_t)e * 2 * I * (H / 32) : p.w2s + (int64_t)e * H * (I / 32)) +
           (int64_t)b_row(tid - TM) * (K / 32);
  float wrow = 0.0f;
  if (!GU && tid < TM) wrow = wsorted[r0 + (tid < nrows ? tid : 0)];

  const int S = K / TK, NCH = S / CHK;
  const bool act = wm * 64 < nrows;   // this wave's rows exist
  int bsel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bsel[j] = GU ? (j < 2 ? wn * 64 + 32 * j : TN / 2 + wn * 64 + 32 * (j - 2)) : wn * 128 + 32 * j;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};

  // scale chunk c (16 bytes of every row) goes straight to scs[c & 1]: lane
  // i of wave w lands at 16 (64 w + i), the thread's own row
  dma16(srow, scs[0] + 1024 * wave);
  issue(abase, 0, offa, lds_addr(la0), wave);
  issue(bbase, 0, offb, lds_addr(lb0), wave);
  issue(abase, (1 < S ? 1 : 0) * TK, offa, lds_addr(la1), wave);
  issue(bbase, (1 < S ? 1 : 0) * TK, offb, lds_addr(lb1), wave);

  // the stage's scale dwords (bytes of this lane's block in 0 and 2)
  int sa[2], sb[4];
  auto scales = [&](int s) {
    const uint8_t *c = scs[(s / CHK) & 1] + 4 * (s % CHK);
#pragma unroll
    for (int i = 0; i < 2; ++i) sa[i] = (int)(*(const uint32_t *)(c + 16 * (wm * 64 + 32 * i + l32)) >> (8 * h));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sb[j] = (int)(*(const uint32_t *)(c + 16 * (TM + bsel[j] + l32)) >> (8 * h));
  };
  // operand fragment of tile row `row` for K-step kk: 16-byte chunks 4 kk + h
  // and 4 kk + 2 + h (the MFMA's two 32-element scale blocks)
  auto frag = [&](const uint8_t *l, int row, int kk) {
    const u32x4 lo = *(const u32x4 *)(l + swz(row, 4 * kk + h));
    const u32x4 hi = *(const u32x4 *)(l + swz(row, 4 * kk + 2 + h));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // one K-step: the two A fragments, then the B fragments one block column
  // ahead of the MFMAs that use them, so LDS reads and MFMAs interleave
  // One K-step: the first MFMA's two fragments are read first (with the
  // stage's scale dwords in K-step 0), the other A fragment and the second
  // B fragment next; each later B fragment is read into the register pair
  // the MFMAs two block columns back have finished with.
  auto kstep = [&](const uint8_t *la, const uint8_t *lb, int kk) {
    i32x8 fa[2], fb[2];
    fa[0] = frag(la, wm * 64 + l32, kk);
    fb[0] = frag(lb, bsel[0] + l32, kk);
    fa[1] = frag(la, wm * 64 + 32 + l32, kk);
    fb[1] = frag(lb, bsel[1] + l32, kk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if constexpr (GU)   // weight rows on the A side (see the epilogue)
          acc[i][j] = kk == 0 ? mfma_mx<0>(fb[j & 1], fa[i], acc[i][j], sb[j], sa[i])
                              : mfma_mx<2>(fb[j & 1], fa[i], acc[i][j], sb[j], sa[i]);
        else
          acc[i][j] = kk == 0 ? mfma_mx<0>(fa[i], fb[j & 1], acc[i][j], sa[i], sb[j])
                              : mfma_mx<2>(fa[i], fb[j & 1], acc[i][j], sa[i], sb[j]);
      if (j + 2 < 4) fb[j & 1] = frag(lb, bsel[j + 2] + l32, kk);
    }
    if (kk == 0)
      __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);               // scales, fa[0], fb[0]
    else
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                // fa[0], fb[0]
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                  // fa[1], fb[1]
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                  // block column 2
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                  // block column 3
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  // stage s: slot (la, lb) readable (loads landed, every wave past the barrier)
  auto ready = [&]() {
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  };
  // stage s computed from (la, lb); stage s+1 waits in (na, nb): after the
  // barrier that follows the stage's last reads, stage s+2 goes to (la, lb)
  auto step = [&](int s, uint8_t *la, uint8_t *lb, uint8_t *na, uint8_t *nb) {
    __builtin_amdgcn_sched_barrier(0);
    // the next chunk's scales go to the buffer chunk s/CHK - 1 used (every
    // wave is past its last read); they land before this stage ends
    if (s % CHK == 0 && s / CHK + 1 < NCH)
      dma16(srow + 16 * (s / CHK + 1), scs[(s / CHK + 1) & 1] + 1024 * wave);
    if (act) {
      scales(s);
      kstep(la, lb, 0);
      __builtin_amdgcn_sched_barrier(0);
      kstep(la, lb, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < S) {
      ready();
      const int t = s + 2 < S ? s + 2 : S - 1;
      issue(abase, t * TK, offa, lds_addr(la), wave);
      issue(bbase, t * TK, offb, lds_addr(lb), wave);
    }
  };
  ready();
  for (int s = 0; s < S; s += 2) {
    step(s, la0, lb0, la1, lb1);
    if (s + 1 < S) step(s + 1, la1, lb1, la0, lb0);
  }
  wait_vmcnt<0>();

  if constexpr (GU) {
    // The gate/up MFMAs take the weight rows as their A operand and the
    // routed rows as B, so a lane's accumulators are one routed row (the
    // lane's column, l32) by 16 h columns: 8q + 4h + (0..3), q = 0..3, of
    // each 32-column block, the other 16 in lane ^ 32.
    // h = silu(g) * u; an MXFP8 block of 32 h columns of one routed row is
    // 16 values of this lane and 16 of lane ^ 32, so its maximum is taken
    // in registers and one exchange.  silu takes the hardware exp2 and
    // reciprocal (a few FP32 ulp, far inside the accumulation tolerance that
    // the re-quantisation check allows), the codes the clamped hardware
    // converter (bit-identical to the encoder); 4 adjacent codes are one
    // dword store.
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = wm * 64 + i * 32 + l32;   // tile row of this lane
        const int cb = c0 + wn * 64 + 32 * jj;  // first h column of the block
        float hv[16];
        float am = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[i][jj][r], u = acc[i][jj + 2][r];
          hv[r] = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          am = fmaxf(am, fabsf(hv[r]));
        }
        am = fmaxf(am, __shfl_xor(am, 32, 64));
        int X = (int)((__builtin_bit_cast(uint32_t, am) >> 23) & 0xFF) - 127 - 8;
        X = X < -127 ? -127 : (X > 127 ? 127 : X);
        const uint32_t sbyte = (uint32_t)(X + 127);   // 0 when amax == 0
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = f32x2_to_e4m3_rne_sat(__builtin_ldexpf(hv[4 * q], -X),
                                                    __builtin_ldexpf(hv[4 * q + 1], -X));
          const uint32_t hi = f32x2_to_e4m3_rne_sat(__builtin_ldexpf(hv[4 * q + 2], -X),
                                                    __builtin_ldexpf(hv[4 * q + 3], -X));
          w4[q] = am == 0.0f ? 0u : ((lo & 0xFFFFu) | (hi << 16));
        }
        if (t < nrows) {
          const int64_t srow2 = r0 + t;
          uint8_t *dq = hq + srow2 * I + cb + 4 * h;
#pragma unroll
          for (int q = 0; q < 4; ++q) *(uint32_t *)(dq + 8 * q) = w4[q];
          if (h == 0) hs[srow2 * (I / 32) + cb / 32] = (uint8_t)sbyte;
          if (p.dbg_gu || p.dbg_h) {
            const int64_t ent = sorted[srow2];
            if (p.dbg_gu) {
              float *d = p.dbg_gu + ent * (2 * I) + cb;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                d[acc_row(r, lane)] = acc[i][jj][r];
                d[I + acc_row(r, lane)] = acc[i][jj + 2][r];
              }
            }
            if (p.dbg_h) {
              uint8_t *d = p.dbg_h + ent * (int64_t)(I + I / 32);
#pragma unroll
              for (int q = 0; q < 4; ++q) *(uint32_t *)(d + cb + 4 * h + 8 * q) = w4[q];
              if (h == 0) d[I + cb / 32] = (uint8_t)sbyte;
            }
          }
        }
      }
  } else {
    // routed rows on the A side: a lane holds one y column (l32) of 16 rows
    if (tid < TM) s_w[tid] = wrow;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + acc_row(r, lane);
        if (row >= nrows) continue;
        const float w = s_w[row];
        float *yrow = y + (int64_t)(r0 + row) * H;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = c0 + wn * 128 + 32 * j + l32;
          if (n < H) yrow[n] = acc[i][j][r] * w;
        }
      }
  }
  // the next item's first loads reuse the slots and the scale buffer
  __syncthreads();
  }
}

}  // namespace t2

// ------------------------------------------- decode-sized MoE (swap-AB)
// With few tokens each expert holds at most a few routed rows, and the call
// streams the active experts' weights once: it is bound by HBM, not by the
// matrix unit.  These two kernels put the weight rows on the MFMA's A side
// (64 per workgroup: two 32-row blocks) and an expert's routed rows (up to 32,
// one block; more are taken 32 at a time) on the B side, each workgroup
// covering the whole of K, so the grids have many workgroups per active
// expert.  Operands go straight from global memory into an LDS ring of SL
// slots (stages of 128 K-elements: 8 KB of weight codes, 4 KB of token codes
// and the rows' E8M0 scale bytes), SL - 1 stages in flight: 6 slots (two
// workgroups per CU) when the grid has at most two workgroups per CU, else 4
// (three per CU, more stages in flight per CU).  Each of the 4 waves
// computes one (block, K-step) pair of every stage; the two waves of a block
// add their sums in a fixed order at the end.
//   k_dec<true>  gate/up: rows [i0, i0+32) of the gate and of the up half of
//                w13[e]; epilogue: GLU and MXFP8 re-quantisation of the 32
//                h columns (one scale block) of each routed row
//   k_dec<false> down: rows [n0, n0+64) of w2[e]; epilogue: times the
//                routing weight, FP32 rows as k_down stores them
// direct-to-LDS load of one dword per lane (lane i at lds + 4 i), tracked by
// the kernel's own vmcnt waits like dma16
__device__ __forceinline__ void dma4(const void *g, const void *lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g),
               "s"(lds_addr(lds))
               : "memory", "m0");
}

constexpr int DROWS = 64;              // weight rows per workgroup
constexpr int DKS = 128;               // K per stage
constexpr int DWB = DROWS * DKS;       // weight code bytes per stage
constexpr int DXB = 32 * DKS;          // token code bytes per stage
constexpr int DSB = 256 * 4;           // scale bytes per stage: one dword per lane of the workgroup
constexpr int DLOADS = 4;              // direct loads per lane per stage

// chunk `chunk` (16 bytes) of 128-byte stage row `row`, XOR-ed with (row / 2) % 8
// so the 16 rows one MFMA fragment read touches at a chunk index cover all
// 64 LDS banks
__device__ __forceinline__ int dk_off(int row, int chunk) {
  return row * DKS + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <bool GU, int DSLOT>
__global__ __launch_bounds__(256) void k_dec(MoeArgs p, const int32_t *meta, const int32_t *sorted,
                                             const float *wsorted, const int32_t *tile_e,
                                             const int32_t *tile_r, const int32_t *tile_n,
                                             uint8_t *hq, uint8_t *hs, float *y) {
  __shared__ __attribute__((aligned(1024))) uint8_t lw[DSLOT * DWB];
  __shared__ __attribute__((aligned(1024))) uint8_t lx[DSLOT * DXB];
  __shared__ __attribute__((aligned(1024))) uint8_t ls[DSLOT * DSB];
  const int tile = blockIdx.y;
  if (tile >= meta[0]) return;
  const int e = tile_e[tile], r0 = tile_r[tile], nrows = tile_n[tile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int H = p.H, I = p.I, K = GU ? H : I, KB = K / 32;
  const int c0 = blockIdx.x * (GU ? 32 : DROWS);   // first h column (gate/up) or hidden column (down)
  const int kstep = wave & 1, blk = wave >> 1;     // this wave's K-step of a stage and weight block

  // weight row q (0..63) of this workgroup, as a row index of w13[e] / w2[e]
  auto wrow = [&](int q) -> int64_t {
    if (GU) return (int64_t)e * 2 * I + (q < 32 ? c0 + q : I + c0 + q - 32);
    return (int64_t)e * H + (c0 + q < H ? c0 + q : H - 1);
  };
  const uint8_t *wq = GU ? p.w13q : p.w2q, *wsc = GU ? p.w13s : p.w2s;
  const uint8_t *xq = GU ? p.xq : hq, *xsc = GU ? p.xs : hs;

  for (int tb = 0; tb < nrows; tb += 32) {
    const int nt = nrows - tb < 32 ? nrows - tb : 32;
    // token (gate/up) or sorted h row (down) of routed row tb + t; rows past
    // the block repeat its first row (their outputs are never stored)
    auto xrow = [&](int t) -> int64_t {
      const int rr = r0 + tb + (t < nt ? t : 0);
      return GU ? (int64_t)(sorted[rr] / p.topk) : (int64_t)rr;
    };
    // this lane's direct loads of a stage: 2 weight chunks, 1 token chunk
    // (16 bytes each; 8 lanes per 128-byte stage row) and one scale dword
    const uint8_t *gw[2], *gx;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * wave + 8 * j + (lane >> 3);
      gw[j] = wq + wrow(row) * K + 16 * ((lane & 7) ^ ((row >> 1) & 7));
    }
    {
      const int row = 8 * wave + (lane >> 3);
      gx = xq + xrow(row) * K + 16 * ((lane & 7) ^ ((row >> 1) & 7));
    }
    // scale dword of the stage: lanes 0..63 weight rows, 64..95 token rows,
    // the rest repeat weight row 0 (never read)
    const uint8_t *gs = tid < 64 ? wsc + wrow(tid) * KB : (tid < 96 ? xsc + xrow(tid - 64) * KB : wsc + wrow(0) * KB);
    auto issue = [&](int s, int slot) {
      const int k0 = s * DKS;
      dma16(gw[0] + k0, lw + slot * DWB + 1024 * (2 * wave));
      dma16(gw[1] + k0, lw + slot * DWB + 1024 * (2 * wave + 1));
      dma16(gx + k0, lx + slot * DXB + 1024 * wave);
      dma4(gs + k0 / 32, ls + slot * DSB + 256 * wave);
    };

    f32x16 acc = {0};
    const int S = K / DKS;
#pragma unroll
    for (int j = 0; j < DSLOT - 1; ++j) issue(j < S ? j : S - 1, j);
    for (int s = 0, slot = 0; s < S; ++s, slot = slot == DSLOT - 1 ? 0 : slot + 1) {
      __builtin_amdgcn_sched_barrier(0);
      // stage s has landed once at most the loads of the DSLOT - 2 stages
      // after it are outstanding (stages past the end reload the last one:
      // never computed)
      wait_vmcnt<(DSLOT - 2) * DLOADS>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // stage s + DSLOT - 1 into the slot stage s - 1 used (every wave is past it)
      issue(s + DSLOT - 1 < S ? s + DSLOT - 1 : S - 1, slot == 0 ? DSLOT - 1 : slot - 1);
      const uint8_t *aw = lw + slot * DWB, *ax = lx + slot * DXB, *as = ls + slot * DSB;
      const int arow = 32 * blk + l32;
      const u32x4 alo = *(const u32x4 *)(aw + dk_off(arow, 4 * kstep + h));
      const u32x4 ahi = *(const u32x4 *)(aw + dk_off(arow, 4 * kstep + 2 + h));
      const u32x4 blo = *(const u32x4 *)(ax + dk_off(l32, 4 * kstep + h));
      const u32x4 bhi = *(const u32x4 *)(ax + dk_off(l32, 4 * kstep + 2 + h));
      // scale of 32-element block (2 kstep + h) of the stage: lane (row, h) of
      // each operand supplies block h of its row
      const int sa = as[4 * arow + 2 * kstep + h], sb = as[4 * (64 + l32) + 2 * kstep + h];
      const i32x8 fa = {(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
      const i32x8 fb = {(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3], (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
      acc = mfma_mx_fp8(fa, fb, acc, sa, sb);
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // block sums: wave 2b + 1's partial added to wave 2b's (K-steps 0 then 1);
    // for gate/up the up block (wave 2) is then handed to wave 0
    float *red = (float *)lw;   // [wave][register][lane]
    if (kstep == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (kstep == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += red[((wave + 1) * 16 + r) * 64 + lane];
    }
    const int t = l32;                 // routed row (token column) of this lane
    if (GU) {
      __syncthreads();
      if (wave == 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(1 * 16 + r) * 64 + lane] = acc[r];
      }
      __syncthreads();
      if (wave == 0) {
        // h = silu(g) * u for columns c0 + row(r) of routed row t; its MXFP8
        // block of 32 columns is this lane's 16 values and lane ^ 32's
        float hv[16];
        float amax = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[r], u = red[(1 * 16 + r) * 64 + lane];
          hv[r] = (g / (1.0f + expf(-g))) * u;
          amax = fmaxf(amax, fabsf(hv[r]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        uint32_t sbyte = 0u;
        int X = 0;
        if (amax != 0.0f) {
          X = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF) - 127 - 8;
          X = X < -127 ? -127 : (X > 127 ? 127 : X);
          sbyte = (uint32_t)(X + 127);
        }
        if (t < nt) {
          const int64_t srow = r0 + tb + t;
          if (p.dbg_gu) {
            float *d = p.dbg_gu + (int64_t)sorted[srow] * (2 * I) + c0;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              d[acc_row(r, lane)] = acc[r];
              d[I + acc_row(r, lane)] = red[(1 * 16 + r) * 64 + lane];
            }
          }
          uint8_t *dq = hq + srow * I + c0;
          uint8_t *dd = p.dbg_h ? p.dbg_h + (int64_t)sorted[srow] * (I + I / 32) : nullptr;
#pragma unroll
          for (int q = 0; q < 4; ++q) {   // registers 4q..4q+3: columns 8q + 4h + 0..3
            uint32_t w4 = 0u;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const uint32_t code = amax == 0.0f ? 0u : f32_to_e4m3_rne_sat(__builtin_ldexpf(hv[4 * q + b], -X));
              w4 |= code << (8 * b);
            }
            *(uint32_t *)(dq + 8 * q + 4 * h) = w4;
            if (dd) *(uint32_t *)(dd + c0 + 8 * q + 4 * h) = w4;
          }
          if (h == 0) {
            hs[srow * (I / 32) + c0 / 32] = (uint8_t)sbyte;
            if (dd) dd[I + c0 / 32] = (uint8_t)sbyte;
          }
        }
      }
    } else if (kstep == 0 && t < nt) {
      // rows c0 + 32 blk + row(r) of y for routed row t, times its routing weight
      const int64_t srow = r0 + tb + t;
      const float w = wsorted[srow];
      float *yrow = y + srow * H + c0 + 32 * blk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 8 * q + 4 * h;
        if (c0 + 32 * blk + n < H)
          *(f32x4 *)(yrow + n) = f32x4{acc[4 * q] * w, acc[4 * q + 1] * w, acc[4 * q + 2] * w, acc[4 * q + 3] * w};
      }
    }
    // the ring (and the reduction area inside it) is reused by the next block
    __syncthreads();
  }
}

// Router top-k (softmax of the logits, the k largest, as the MoE
// configuration routes) of one token by one wave: expert e in lane e % 64,
// register e / 64.  The softmax is taken in FP32 (max, exp, a butterfly sum
// that leaves every lane the same value, one division per weight); the k
// experts are chosen on the logits, which orders them as the exact
// probabilities (equal logits: the lower id first).  Slot j's id and weight
// go to ids[j], w[j] and, when given, to the LDS copies lids[j], lw[j].
template <int PER>
__device__ __forceinline__ void load_logits(const float *row, int E, int lane, float (&v)[PER]) {
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int e = lane + 64 * q;
    v[q] = e < E ? row[e] : -__builtin_inff();
  }
}

// the same on logits already loaded (this lane's v[q] = logit lane + 64 q)
template <int PER>
__device__ __forceinline__ void route_loaded(float (&v)[PER], int E, int topk, int lane,
                                             int32_t *ids, float *w, int32_t *lids, float *lw) {
  float ex[PER];
  float m = -__builtin_inff();
#pragma unroll
  for (int q = 0; q < PER; ++q) m = fmaxf(m, v[q]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    ex[q] = lane + 64 * q < E ? expf(v[q] - m) : 0.0f;
    s += ex[q];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  for (int j = 0; j < topk; ++j) {
    // the largest remaining logit, lowest id on equal values
    float bv = -__builtin_inff();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = lane + 64 * q;
      if (e < E && (v[q] > bv || (v[q] == bv && e < be))) {
        bv = v[q];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if (lane == (be & 63)) {
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (q == be >> 6) {
          const float p = ex[q] / s;
          ids[j] = be;
          w[j] = p;
          if (lids) {
            lids[j] = be;
            lw[j] = p;
          }
          v[q] = -__builtin_inff();   // taken (finite logits: never chosen again)
        }
    }
  }
}

template <int PER>
__device__ __forceinline__ void route_token(const float *row, int E, int topk, int lane,
                                            int32_t *ids, float *w, int32_t *lids, float *lw) {
  float v[PER];
  load_logits<PER>(row, E, lane, v);
  route_loaded<PER>(v, E, topk, lane, ids, w, lids, lw);
}

// the router alone: one wave per token
template <int PER>
__global__ __launch_bounds__(256) void k_topk_softmax(const float *logits, int T, int E, int topk,
                                                      int32_t *ids, float *w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<PER>(logits + (int64_t)t * E, E, topk, lane, ids + (int64_t)t * topk,
                   w + (int64_t)t * topk, nullptr, nullptr);
}

// Route prep from the router logits (the four-kernel routing's k_count with
// the router fused in): each workgroup routes RT_TOK tokens (one wave per
// token at a time), writes their ids and weights, then counts its entries per
// expert in LDS, reserves each expert's run of ranks with one global atomic,
// and writes each entry's rank -- what k_topk_softmax then k_count compute,
// without the ids' round trip through a second launch.
constexpr int RT_TOK = 64;   // tokens per workgroup (16 waves x 4)
template <int PER>
__global__ __launch_bounds__(1024) void k_count_logits(const float *logits, int T, int E, int topk,
                                                      int32_t *ids, float *tw, uint32_t *counts,
                                                      int32_t *rank) {
  __shared__ uint32_t s_cnt[1024], s_base[1024];
  __shared__ int32_t s_ids[RT_TOK * 16];   // topk <= 16
  __shared__ float s_w[RT_TOK * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TOK;
  const int nt = T - t0 < RT_TOK ? T - t0 : RT_TOK;
  for (int e = tid; e < E; e += 1024) s_cnt[e] = 0u;
  // this wave's tokens i = wave + 16 q: every logit requested before the
  // first is used (one memory latency, not one per token)
  constexpr int TPW = RT_TOK / 16;
  float v[TPW][PER];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int i = wave + 16 * q;
    load_logits<PER>(logits + (int64_t)(t0 + (i < nt ? i : 0)) * E, E, lane, v[q]);
  }
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int i = wave + 16 * q;
    if (i < nt) {
      const int64_t t = t0 + i;
      route_loaded<PER>(v[q], E, topk, lane, ids + t * topk, tw + t * topk, s_ids + i * topk,
                        s_w + i * topk);
    }
  }
  __syncthreads();
  const int n = nt * topk;            // entries of this workgroup (at most 1024)
  const int e = tid < n ? s_ids[tid] : -1;
  const uint32_t lr = tid < n ? atomicAdd(&s_cnt[e], 1u) : 0u;
  __syncthreads();
  for (int x = tid; x < E; x += 1024)
    if (s_cnt[x] != 0u) s_base[x] = atomicAdd(&counts[CSTRIDE * x], s_cnt[x]);
  __syncthreads();
  if (tid < n) rank[(int64_t)t0 * topk + tid] = (int32_t)(s_base[e] + lr);
}

// one thread per (token, 4 columns): slots summed in order 0..topk-1; every
// slot's row index, then every row, is requested before the first add
__global__ void k_combine(const float *y, const int32_t *pos, int T, int H, int topk,
                          uint16_t *out) {
  constexpr int MAXK = 16;   // topk limit of the entry point
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_t = H / 4;
  if (q >= (int64_t)T * per_t) return;
  const int t = (int)(q / per_t), c = (int)(q % per_t) * 4;
  int r[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) r[j] = j < topk ? pos[(int64_t)t * topk + j] : -1;
  f32x4 v[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j)
    v[j] = r[j] >= 0 ? *(const f32x4 *)(y + (int64_t)r[j] * H + c) : f32x4{0, 0, 0, 0};
  f32x4 a = {0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < MAXK; ++j) a = r[j] >= 0 ? a + v[j] : a;
  *(u32x2 *)(out + (int64_t)t * H + c) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
}

// Decode-sized routing (R <= 1024 entries, E <= 1024 experts) in one
// workgroup: what k_prep, k_count, k_scan and k_scatter do, with the expert
// counters and both scans in LDS, so the call spends one launch on it.  With
// LOGITS the router runs first in the same workgroup (one wave per token, as
// k_topk_softmax): it writes the T tokens' ids and weights to `ids` / `tw`
// (outputs then) and keeps them in LDS for the counting.
template <bool LOGITS, int PER>
__global__ __launch_bounds__(1024) void k_route_small(const int32_t *ids, const float *tw, int R,
                                                      int E, int32_t *offs, int32_t *meta,
                                                      int32_t *tile_e, int32_t *tile_r,
                                                      int32_t *tile_n, int32_t *pos,
                                                      int32_t *sorted, float *wsorted,
                                                      const float *logits, int T, int topk) {
  __shared__ uint32_t s_cnt[1024];
  __shared__ int s_rows[1024], s_tiles[1024];
  __shared__ int32_t s_ids[LOGITS ? 1024 : 1];
  __shared__ float s_w[LOGITS ? 1024 : 1];
  const int tid = threadIdx.x;
  s_cnt[tid] = 0u;
  if constexpr (LOGITS) {
    const int lane = tid & 63;
    for (int t = tid >> 6; t < T; t += 16)
      route_token<PER>(logits + (int64_t)t * E, E, topk, lane, (int32_t *)ids + t * topk,
                       (float *)tw + t * topk, s_ids + t * topk, s_w + t * topk);
  }
  __syncthreads();
  const int e = tid < R ? (LOGITS ? s_ids[tid] : ids[tid]) : -1;
  const bool ok = e >= 0 && e < E;
  const uint32_t rk = ok ? atomicAdd(&s_cnt[e], 1u) : 0u;   // rank within the expert
  __syncthreads();
  // inclusive scans over experts (thread = expert) of rows and 128-row tiles
  const int c = tid < E ? (int)s_cnt[tid] : 0, nt = (c + BM - 1) / BM;
  s_rows[tid] = c;
  s_tiles[tid] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int ar = tid >= o ? s_rows[tid - o] : 0, at = tid >= o ? s_tiles[tid - o] : 0;
    __syncthreads();
    s_rows[tid] += ar;
    s_tiles[tid] += at;
    __syncthreads();
  }
  if (tid == 1023) meta[0] = s_tiles[1023];
  if (tid < E) {
    const int rb = s_rows[tid] - c, tb = s_tiles[tid] - nt;
    offs[tid] = rb;
    for (int q = 0; q < nt; ++q) {
      tile_e[tb + q] = tid;
      tile_r[tb + q] = rb + q * BM;
      tile_n[tb + q] = c - q * BM < BM ? c - q * BM : BM;
    }
  }
  if (tid < R) {
    if (ok) {
      const int p = s_rows[e] - (int)s_cnt[e] + (int)rk;
      pos[tid] = p;
      sorted[p] = tid;
      wsorted[p] = LOGITS ? s_w[tid] : tw[tid];
    } else {
      pos[tid] = -1;
    }
  }
}

}  // namespace

// the decode-sized kernels serve up to 32 tokens when both K dimensions are
// whole stages (an expert then has at most 32 rows unless a token names it
// twice; such rows are taken 32 at a time)
static int moe_cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 256;
    return cus;
  }();
  return n;
}

// the 256 x 256 grouped GEMMs: scale rows in 16-byte chunks (H, I multiples
// of 512), 128 h columns per gate/up tile, and every row offset of an
// operand within 32 bits
static bool mx256_path(const MoeArgs &p) {
  const int64_t R = (int64_t)p.T * p.topk, lim = (int64_t)1 << 32;
  return p.H % 512 == 0 && p.I % 512 == 0 && (int64_t)p.T * p.H < lim && R * p.I < lim &&
         (int64_t)2 * p.I * p.H < lim;
}

static bool dec_path(const MoeArgs &p) {
  return p.T <= 32 && (int64_t)p.T * p.topk <= 1024 && p.H % DKS == 0 && p.I % DKS == 0;
}

size_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  return layout(T, H, I, E, topk).total;
}

hipError_t launch_moe(const MoeArgs &p, hipStream_t stream) {
  const Layout L = layout(p.T, p.H, p.I, p.E, p.topk);
  char *w = (char *)p.ws;
  uint32_t *counts = (uint32_t *)(w + L.counts);
  int32_t *meta = (int32_t *)(w + L.meta);
  int32_t *sorted = (int32_t *)(w + L.sorted);
  int32_t *tile_e = (int32_t *)(w + L.tile_e);
  int32_t *tile_r = (int32_t *)(w + L.tile_r);
  int32_t *tile_n = (int32_t *)(w + L.tile_n);
  uint8_t *hq = (uint8_t *)(w + L.hq);
  uint8_t *hs = (uint8_t *)(w + L.hs);
  int32_t *pos = (int32_t *)(w + L.pos);
  float *y = (float *)(w + L.y);
  const int64_t TH4 = (int64_t)p.T * (p.H / 4);

  int32_t *offs = (int32_t *)(w + L.offs);
  float *wsorted = (float *)(w + L.wsorted);
  if (dec_path(p)) {
    // decode-sized: one routing launch; every active tile has at least one
    // row, so at most R tiles
    if (!p.logits)
      hipLaunchKernelGGL((k_route_small<false, 1>), dim3(1), dim3(1024), 0, stream, p.ids, p.tw, L.R,
                         p.E, offs, meta, tile_e, tile_r, tile_n, pos, sorted, wsorted, nullptr, p.T,
                         p.topk);
    else if (p.E <= 64)
      hipLaunchKernelGGL((k_route_small<true, 1>), dim3(1), dim3(1024), 0, stream, p.ids, p.tw, L.R,
                         p.E, offs, meta, tile_e, tile_r, tile_n, pos, sorted, wsorted, p.logits,
                         p.T, p.topk);
    else if (p.E <= 256)
      hipLaunchKernelGGL((k_route_small<true, 4>), dim3(1), dim3(1024), 0, stream, p.ids, p.tw, L.R,
                         p.E, offs, meta, tile_e, tile_r, tile_n, pos, sorted, wsorted, p.logits,
                         p.T, p.topk);
    else
      hipLaunchKernelGGL((k_route_small<true, 16>), dim3(1), dim3(1024), 0, stream, p.ids, p.tw,
                         L.R, p.E, offs, meta, tile_e, tile_r, tile_n, pos, sorted, wsorted,
                         p.logits, p.T, p.topk);
    const unsigned ty = (unsigned)(L.maxtiles < L.R ? L.maxtiles : L.R);
    const dim3 gg(p.I / 32, ty), gd(p.H / DROWS, ty);
    // at most two active workgroups per CU (of 256): the deeper ring
    const int64_t te = p.E < L.R ? p.E : L.R;   // active tiles, without repeated experts
    if (te * (p.I / 32) <= 512)
      hipLaunchKernelGGL((k_dec<true, 6>), gg, dim3(256), 0, stream, p, meta, sorted, wsorted,
                         tile_e, tile_r, tile_n, hq, hs, y);
    else
      hipLaunchKernelGGL((k_dec<true, 4>), gg, dim3(256), 0, stream, p, meta, sorted, wsorted,
                         tile_e, tile_r, tile_n, hq, hs, y);
    if (te * (p.H / DROWS) <= 512)
      hipLaunchKernelGGL((k_dec<false, 6>), gd, dim3(256), 0, stream, p, meta, sorted, wsorted,
                         tile_e, tile_r, tile_n, hq, hs, y);
    else
      hipLaunchKernelGGL((k_dec<false, 4>), gd, dim3(256), 0, stream, p, meta, sorted, wsorted,
                         tile_e, tile_r, tile_n, hq, hs, y);
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((TH4 + 255) / 256)), dim3(256), 0, stream, y,
                       pos, p.T, p.H, p.topk, p.out);
    return hipGetLastError();
  }
  const int rb = (L.R + 255) / 256;
  hipLaunchKernelGGL(k_prep, dim3((p.E + 255) / 256), dim3(256), 0, stream, counts, p.E);
  if (!p.logits) {
    hipLaunchKernelGGL(k_count, dim3((L.R + 1023) / 1024), dim3(1024), 0, stream, p.ids, L.R, p.E,
                       counts, pos);
  } else {
    // the router fused into the count: ids and weights written here
    const dim3 gr((unsigned)((p.T + RT_TOK - 1) / RT_TOK));
    int32_t *ids = (int32_t *)p.ids;
    float *tw = (float *)p.tw;
    if (p.E <= 64)
      hipLaunchKernelGGL(k_count_logits<1>, gr, dim3(1024), 0, stream, p.logits, p.T, p.E, p.topk,
                         ids, tw, counts, pos);
    else if (p.E <= 256)
      hipLaunchKernelGGL(k_count_logits<4>, gr, dim3(1024), 0, stream, p.logits, p.T, p.E, p.topk,
                         ids, tw, counts, pos);
    else
      hipLaunchKernelGGL(k_count_logits<16>, gr, dim3(1024), 0, stream, p.logits, p.T, p.E, p.topk,
                         ids, tw, counts, pos);
  }
  const bool big = mx256_path(p);
  if (big)
    hipLaunchKernelGGL(k_scan<t2::TM>, dim3(1), dim3(256), 0, stream, counts, p.E, offs, meta,
                       tile_e, tile_r, tile_n);
  else
    hipLaunchKernelGGL(k_scan<BM>, dim3(1), dim3(256), 0, stream, counts, p.E, offs, meta, tile_e,
                       tile_r, tile_n);
  hipLaunchKernelGGL(k_scatter, dim3(rb), dim3(256), 0, stream, p.ids, p.tw, L.R, offs, pos, sorted,
                     wsorted);
  if (big) {
    // one workgroup per CU (the kernels walk their items)
    const dim3 grid(moe_cu_count());
    hipLaunchKernelGGL(t2::k_mx256<true>, grid, dim3(t2::NT), 0, stream, p, meta, sorted, wsorted,
                       tile_e, tile_r, tile_n, hq, hs, y);
    hipLaunchKernelGGL(t2::k_mx256<false>, grid, dim3(t2::NT), 0, stream, p, meta, sorted, wsorted,
                       tile_e, tile_r, tile_n, hq, hs, y);
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((TH4 + 255) / 256)), dim3(256), 0, stream, y,
                       pos, p.T, p.H, p.topk, p.out);
    return hipGetLastError();
  }
  // scale rows of 16-byte multiples (K % 512 == 0) take the chunked scale loads
  const dim3 gg(p.I / BNI, L.maxtiles), gd((p.H + BNH - 1) / BNH, L.maxtiles);
  if (p.H % 512 == 0)
    hipLaunchKernelGGL(k_gateup<true>, gg, dim3(256), 0, stream, p, meta, sorted, tile_e, tile_r,
                       tile_n, hq, hs);
  else
    hipLaunchKernelGGL(k_gateup<false>, gg, dim3(256), 0, stream, p, meta, sorted, tile_e, tile_r,
                       tile_n, hq, hs);
  if (p.I % 512 == 0)
    hipLaunchKernelGGL(k_down<true>, gd, dim3(256), 0, stream, p, meta, wsorted, tile_e, tile_r,
                       tile_n, hq, hs, y);
  else
    hipLaunchKernelGGL(k_down<false>, gd, dim3(256), 0, stream, p, meta, wsorted, tile_e, tile_r,
                       tile_n, hq, hs, y);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((TH4 + 255) / 256)), dim3(256), 0, stream, y, pos,
                     p.T, p.H, p.topk, p.out);
  return hipGetLastError();
}

}  // namespace mg

namespace mg {

size_t moe4_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int64_t topk) {
  return layout(T, H, I, E, topk, true).total;
}

// NVFP4 MoE: the routing and the combine of the MXFP8 MoE around the grouped
// W4A4 GEMMs of moe4.hip
hipError_t launch_moe4(const Moe4Args &p, hipStream_t stream) {
  const Layout L = layout(p.T, p.H, p.I, p.E, p.topk, true);
  char *w = (char *)p.ws;
  uint32_t *counts = (uint32_t *)(w + L.counts);
  int32_t *offs = (int32_t *)(w + L.offs);
  int32_t *meta = (int32_t *)(w + L.meta);
  int32_t *sorted = (int32_t *)(w + L.sorted);
  int32_t *pos = (int32_t *)(w + L.pos);
  float *wsorted = (float *)(w + L.wsorted);
  int32_t *tile_e = (int32_t *)(w + L.tile_e);
  int32_t *tile_r = (int32_t *)(w + L.tile_r);
  int32_t *tile_n = (int32_t *)(w + L.tile_n);
  uint8_t *hq = (uint8_t *)(w + L.hq);
  uint8_t *hs = (uint8_t *)(w + L.hs);
  float *y = (float *)(w + L.y);
  const int64_t TH4 = (int64_t)p.T * (p.H / 4);
  if (L.R <= 1024) {
    hipLaunchKernelGGL((k_route_small<false, 1>), dim3(1), dim3(1024), 0, stream, p.ids, p.tw, L.R,
                       p.E, offs, meta, tile_e, tile_r, tile_n, pos, sorted, wsorted, nullptr, p.T,
                       p.topk);
  } else {
    const int rb = (L.R + 255) / 256;
    hipLaunchKernelGGL(k_prep, dim3((p.E + 255) / 256), dim3(256), 0, stream, counts, p.E);
    hipLaunchKernelGGL(k_count, dim3((L.R + 1023) / 1024), dim3(1024), 0, stream, p.ids, L.R,
                       p.E, counts, pos);
    hipLaunchKernelGGL(k_scan<BM>, dim3(1), dim3(256), 0, stream, counts, p.E, offs, meta, tile_e,
                       tile_r, tile_n);
    hipLaunchKernelGGL(k_scatter, dim3(rb), dim3(256), 0, stream, p.ids, p.tw, L.R, offs, pos,
                       sorted, wsorted);
  }
  // every active tile has at least one row: at most R tiles
  const int ty = L.maxtiles < L.R ? L.maxtiles : L.R;
  hipError_t e = launch_moe4_gemms(p, meta, sorted, wsorted, tile_e, tile_r, tile_n, ty, hq, hs,
                                   y, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((TH4 + 255) / 256)), dim3(256), 0, stream, y,
                     pos, p.T, p.H, p.topk, p.out);
  return hipGetLastError();
}

}  // namespace mg

namespace mg {

hipError_t launch_topk_softmax(const float *logits, int T, int E, int topk, int32_t *ids,
                               float *w, hipStream_t stream) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk_softmax<1>, grid, block, 0, stream, logits, T, E, topk, ids, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk_softmax<4>, grid, block, 0, stream, logits, T, E, topk, ids, w);
  else
    hipLaunchKernelGGL(k_topk_softmax<16>, grid, block, 0, stream, logits, T, E, topk, ids, w);
  return hipGetLastError();
}

}  // namespace mg
