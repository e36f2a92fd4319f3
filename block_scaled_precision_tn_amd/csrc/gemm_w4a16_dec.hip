// gemm_w4a16_dec.hip -- small-M (decode) W4A16 on gfx950: BF16 activations
// under NVFP4 weights, the weights widened to BF16 in registers and run on
// the BF16 MFMA (metrale_circuit hardware::exec module description: BF16
// activations take the BF16 MMA with the weight format widened in registers).
//
// With few tokens the call streams the weight (N*K/2 code bytes + N*K/16
// scale bytes) once, so it is arranged for HBM:
//   * swap-AB: weight rows are the MFMA's B side (lane column = weight row),
//     tokens its A side in blocks of 32 (lanes of token rows >= M read row 0;
//     those MFMA rows are never stored);
//   * split-K: a workgroup covers 64 weight rows of one K range (1024
//     elements up to 16 tokens, 512 above); its four waves are two 32-row
//     blocks x the two halves of the range.  Each lane loads its own bytes
//     straight into registers -- per 64-element chunk of its half, 16 code
//     bytes (32 elements) and the 2 scale bytes of their two groups -- all
//     issued up front, after the range's token rows (direct to LDS), so the
//     first chunks are computed while the rest are still arriving;
//   * one v_permlane32_swap per two dwords turns the lane pair (row, half 0)
//     and (row, half 1) holding 64 consecutive elements into four MFMA
//     operands of one 16-element group each (lane half h supplies elements
//     8h .. 8h+7 of the group), so every MFMA sees a single group scale per
//     weight row;
//   * the group scale is applied in one of two ways:
//       - up to 16 tokens: v_cvt_scalef32_pk_bf16_fp4 widens two codes per
//         instruction and applies the power of two 2^E of the scale's FP32
//         value (the converter uses only its scale operand's exponent), one
//         MFMA per group with a zero accumulator, then the rest of the scale,
//         2 * frexp_mant(s) in [1, 2) (exact in FP32), by one FP32 fused
//         multiply-add per accumulator register that holds a real token
//         (1, 4 or 8 of the 16);
//       - more tokens: each code pair is widened exactly to FP32
//         (v_cvt_scalef32_pk_f32_fp4, scale 1), multiplied by the scale
//         (exact) and packed to BF16 (v_cvt_pk_bf16_f32, exact: at most 6
//         significant bits), and the MFMAs accumulate directly;
//     the FP32 tensor scale S_w (and the first way's factor 2) is applied
//     once per output;
//   * the splits are summed by a second kernel, in split order 0..ks-1
//     (run-to-run bit-identical), which applies S_w (and the first way's
//     factor 2).  (Summing them in the kernel, by each tile's last workgroup
//     to finish, was measured slower: the partials then have to reach the
//     device's coherence point and the last workgroup's ticket and reads add
//     a chain of round trips at the end of the stream.)
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int MAXM = 128;      // tokens per launch (up to four blocks of 32)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// K range of one workgroup: 1024 elements for up to 16 tokens, 512 above
__host__ __device__ constexpr int range_of(int m) { return m <= 16 ? 1024 : 512; }

// codes of dword w (byte i = elements 2i, 2i+1 in its low, high nibble) as 8
// BF16 in element order, each = e2m1 * 2^E where 2^E is the power of two of
// s's FP32 exponent field
__device__ __forceinline__ u32x4 widen8_pow2(uint32_t w, float s) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
}

// the same 8 codes as BF16 of e2m1 * s, exact
__device__ __forceinline__ uint32_t pair_scaled(f32x2 x, float s) {
  x[0] *= s;
  x[1] *= s;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ u32x4 widen8_exact(uint32_t w, float s) {
  return u32x4{pair_scaled(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), s),
               pair_scaled(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), s),
               pair_scaled(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), s),
               pair_scaled(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), s)};
}

// R > 0: the power-of-two widening with R live accumulator registers per
// lane (R = 1: one token, 4: up to 8, 8: up to 16); R = 0: exact widening,
// TB token blocks of 32.  NB blocks of 32 weight rows per workgroup (2 NB
// waves: NB blocks x the two halves of the range); more rows per workgroup
// spread the token rows it stages over more weight rows.  WIDE: K % (256 or
// 128) == 0, so each lane fetches the scale bytes of its whole range with
// one 16- or 8-byte load.  Dynamic LDS: max(rows * TROW, NB * TB * 4096)
// bytes.
template <int R, int TB, bool WIDE, int NB>
__global__ __launch_bounds__(128 * NB) void w4a16_dec_kernel(Bf16Args p, int ks, float *part) {
  constexpr int DK = range_of(R > 0 ? 16 : 17);
  constexpr int HK = DK / 2, CH = HK / 64, TROW = 2 * DK + 16, CPR = DK / 8;
  constexpr int LIVE = R > 0 ? R : 16;   // accumulator registers that can hold tokens
  constexpr int NW = 2 * NB, DN = 32 * NB;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int blk = wave % NB, kh = wave / NB;
  const int nt = blockIdx.x / ks, kc = blockIdx.x % ks;
  const int n0 = nt * DN, k0 = kc * DK;
  const int klen = p.K - k0 < DK ? p.K - k0 : DK;   // a multiple of 32
  const int rows = p.M < 32 * TB ? p.M : 32 * TB;   // token rows held in LDS

  // 1. the range's token rows into LDS, direct: a wave instruction moves 64
  // consecutive 16-byte pieces of one row; pieces past klen are zeroed by
  // their own lane instead (they meet zero weights, and zero keeps the
  // products finite)
  int dma = 0;
  for (int j = wave; j < rows * (CPR / 64); j += NW, ++dma) {
    const int t = j / (CPR / 64), c = (j % (CPR / 64)) * 64 + lane;
    uint8_t *dst = lds + t * TROW + 1024 * (j % (CPR / 64));
    if (8 * c < klen)
      dma16(p.a + (int64_t)t * p.K + k0 + 8 * c, dst);
    else
      *(u32x4 *)(dst + 16 * lane) = u32x4{0, 0, 0, 0};
  }

  // 2. this lane's weight bytes: chunk c holds elements kw + 64c + 32h .. +31
  // of row n (rows past N re-read row N-1 and are never stored; elements
  // past K read an in-bounds address and are masked).  The scale bytes come
  // first: the compiler widens narrow loads right after they land, and that
  // wait then does not cover the code bytes.
  const int nr = n0 + 32 * blk + l32;
  const int n = nr < p.N ? nr : p.N - 1;
  const int kw = k0 + kh * HK;
  const int G = p.K / 16;
  const uint8_t *srow = p.ws + (int64_t)n * G;
  u32x4 sv = {0, 0, 0, 0};   // WIDE: groups kw/16 + 2CH h .. + 2CH - 1 (CH/2 dwords)
  uint16_t sn[CH];           // otherwise: groups (kw + 64c + 32h)/16 + {0, 1}
  if constexpr (WIDE) {
    // a lane's 2CH-byte window is aligned and lies wholly inside or wholly
    // past the row (G is a multiple of 2CH); past it, any in-bounds window
    // (its chunks are dead)
    int g = kw / 16 + 2 * CH * h;
    g = g < G ? g : G - 2 * CH;
    if constexpr (CH == 8) {
      sv = *(const u32x4 *)(srow + g);
    } else {
      const u32x2 v = *(const u32x2 *)(srow + g);
      sv[0] = v[0];
      sv[1] = v[1];
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = kw + 64 * c + 32 * h;
      sn[c] = *(const uint16_t *)(srow + (k < p.K ? k : p.K - 32) / 16);
    }
  }
  u32x4 code[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = kw + 64 * c + 32 * h;
    const int kk = k < p.K ? k : p.K - 32;
    code[c] = *(const u32x4 *)((const uint8_t *)p.w + (int64_t)n * (p.K / 2) + kk / 2);
  }

  // 3. own token loads landed (the weight loads issued after them may still
  // be in flight), then every wave's
  if (dma > 0) {
    if constexpr (WIDE)
      wait_vmcnt<CH + 1>();
    else
      wait_vmcnt<2 * CH>();
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();

  f32x16 acc[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) acc[b] = f32x16{0};
  const uint8_t *arow[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int t = 32 * b + l32;
    arow[b] = lds + (t < rows ? t : 0) * TROW;
  }
  uint32_t s_hi[CH / 2];   // WIDE: the second half's scale dwords, kept from the swaps
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    // keep each chunk's work after the previous chunk's, so the compiler's
    // wait for chunk c's loads does not also wait for later chunks
    __builtin_amdgcn_sched_barrier(0);
    const int kl = kh * HK + 64 * c;   // chunk start within the range
    const bool live = kl + 32 * h < klen;
    const u32x4 cw = live ? code[c] : u32x4{0, 0, 0, 0};
    // the chunk's four group scales at every lane of the row: byte i = group i
    uint32_t s4;
    if constexpr (WIDE) {
      if (c < CH / 2) {
        const auto r = __builtin_amdgcn_permlane32_swap(sv[c], sv[c], false, false);
        s4 = r[0];
        s_hi[c] = r[1];
      } else {
        s4 = s_hi[c - CH / 2];
      }
    } else {
      const uint32_t x = sn[c];
      const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      s4 = r[0] | (r[1] << 16);
    }
    // groups of a dead half: scale 0 (their codes are zero too)
    s4 &= kl + 32 < klen ? 0xFFFFFFFFu : (kl < klen ? 0xFFFFu : 0u);
    // group operands: [0] = group 0 (from half 0), [1] = group 2 (half 1)
    const auto g02 = __builtin_amdgcn_permlane32_swap(cw[0], cw[1], false, false);
    const auto g13 = __builtin_amdgcn_permlane32_swap(cw[2], cw[3], false, false);
    const f32x2 s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s4, 1.0f, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s4, 1.0f, true);
    const uint32_t wg[4] = {g02[0], g13[0], g02[1], g13[1]};
    const float sg[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (R > 0) {
        const u32x4 wv = widen8_pow2(wg[g], sg[g]);
        const float f = __builtin_amdgcn_frexp_mantf(sg[g]);
        const u32x4 av = *(const u32x4 *)(arow[0] + 2 * (kl + 16 * g + 8 * h));
        const f32x16 t = mfma_bf16(av, wv, f32x16{0});
#pragma unroll
        for (int r = 0; r < R; ++r) acc[0][r] = __builtin_fmaf(f, t[r], acc[0][r]);
      } else {
        const u32x4 wv = widen8_exact(wg[g], sg[g]);
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const u32x4 av = *(const u32x4 *)(arow[b] + 2 * (kl + 16 * g + 8 * h));
          acc[b] = mfma_bf16(av, wv, acc[b]);
        }
      }
    }
  }

  // 4. the two halves of the range, added in a fixed order (half 0 + half 1),
  // into this split's partial
  __syncthreads();
  float *xch = (float *)lds;   // [blk][b][r][lane]
  if (kh == 1) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int r = 0; r < LIVE; ++r) xch[((blk * TB + b) * 16 + r) * 64 + lane] = acc[b][r];
  }
  __syncthreads();
  if (kh == 0 && nr < p.N) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int r = 0; r < LIVE; ++r) {
        const int t = 32 * b + acc_row(r, lane);
        const float v = acc[b][r] + xch[((blk * TB + b) * 16 + r) * 64 + lane];
        if (t < p.M) part[((int64_t)kc * p.M + t) * p.N + nr] = v;
      }
  }
}

// C[t,n] = (sum over splits 0..ks-1, in order, of part[s,t,n]) * post * S_w
__global__ __launch_bounds__(256) void w4a16_dec_reduce(Bf16Args p, int ks, const float *part,
                                                        float post) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t mn = (int64_t)p.M * p.N;
  if (i >= mn) return;
  constexpr int PRE = 32;   // partials requested before the ordered sum
  float v = 0.0f;
  for (int s0 = 0; s0 < ks; s0 += PRE) {
    float x[PRE];
#pragma unroll
    for (int j = 0; j < PRE; ++j)
      if (s0 + j < ks) x[j] = part[(int64_t)(s0 + j) * mn + i];
#pragma unroll
    for (int j = 0; j < PRE; ++j)
      if (s0 + j < ks) v += x[j];
  }
  v *= post * *p.Sw;
  if (p.out_f32)
    ((float *)p.C)[i] = v;
  else
    ((uint16_t *)p.C)[i] = (uint16_t)f32_to_bf16_rne(v);
}

template <int R, int TB, bool WIDE, int NB>
hipError_t launch_one(const Bf16Args &p, int ks, float *part, hipStream_t stream) {
  constexpr int DK = range_of(R > 0 ? 16 : 17), TROW = 2 * DK + 16, DN = 32 * NB;
  constexpr int XCH = NB * TB * 4096;   // the range halves' exchange
  constexpr int MAXL = 32 * TB * TROW > XCH ? 32 * TB * TROW : XCH;
  const int rows = p.M < 32 * TB ? p.M : 32 * TB;
  const size_t lds = (size_t)(rows * TROW > XCH ? rows * TROW : XCH);
  if constexpr (MAXL > 65536) {
    // more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
    static const hipError_t attr =
        hipFuncSetAttribute((const void *)w4a16_dec_kernel<R, TB, WIDE, NB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, MAXL);
    if (attr != hipSuccess) return attr;
  }
  const dim3 grid((unsigned)(((p.N + DN - 1) / DN) * ks));
  hipLaunchKernelGGL((w4a16_dec_kernel<R, TB, WIDE, NB>), grid, dim3(128 * NB), lds, stream, p, ks,
                     part);
  const int64_t mn = (int64_t)p.M * p.N;
  hipLaunchKernelGGL(w4a16_dec_reduce, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream, p,
                     ks, (const float *)part, R > 0 ? 2.0f : 1.0f);
  return hipGetLastError();
}

template <int R, int TB, int NB = 2>
hipError_t launch_sel(const Bf16Args &p, int ks, float *part, hipStream_t stream) {
  constexpr int CH = range_of(R > 0 ? 16 : 17) / 128;
  if ((p.K / 16) % (2 * CH) == 0) return launch_one<R, TB, true, NB>(p, ks, part, stream);
  return launch_one<R, TB, false, NB>(p, ks, part, stream);
}

}  // namespace

size_t w4a16_dec_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M > W4A16_DEC_MAX_M) return 0;
  const int64_t mb = M < MAXM ? M : MAXM;
  const int64_t ks = (K + range_of((int)mb) - 1) / range_of((int)mb);
  return (size_t)ks * (size_t)mb * (size_t)N * sizeof(float);
}

hipError_t launch_w4a16_dec(const Bf16Args &p0, void *ws, hipStream_t stream) {
  float *part = (float *)ws;
  for (int m0 = 0; m0 < p0.M; m0 += MAXM) {
    Bf16Args p = p0;
    p.M = p0.M - m0 < MAXM ? p0.M - m0 : MAXM;
    p.a = p0.a + (int64_t)m0 * p0.K;
    p.C = (char *)p0.C + (int64_t)m0 * p0.N * (p0.out_f32 ? 4 : 2);
    const int ks = (p.K + range_of(p.M) - 1) / range_of(p.M);
    hipError_t e;
    if (p.M == 1)
      e = launch_sel<1, 1>(p, ks, part, stream);
    else if (p.M <= 8)
      e = launch_sel<4, 1>(p, ks, part, stream);
    else if (p.M <= 16)
      e = launch_sel<8, 1>(p, ks, part, stream);
    else if (p.M <= 32)
      e = launch_sel<0, 1>(p, ks, part, stream);
    else if (p.M <= 64)
      e = launch_sel<0, 2>(p, ks, part, stream);
    else   // 128 weight rows per workgroup: the 128 staged token rows serve twice the weight
      e = launch_sel<0, 4, 4>(p, ks, part, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mg
