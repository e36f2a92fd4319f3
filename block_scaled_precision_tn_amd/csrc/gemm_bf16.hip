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
// Workgroup: 256 threads (4 waves, 2x2), tile 128 x 128 x 64, wave tile
// 64 x 64 = 2 x 2 blocks of v_mfma_f32_32x32x16_bf16.  Operands are staged
// through LDS (double-buffered) in 16-byte chunks whose position within a
// 128-byte row is XOR-swizzled by the row index, so the MFMA fragment reads
// (32 rows x one chunk) hit distinct banks.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS row (64 BF16)

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ (row & 7)) << 4); }

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

template <bool WQ>
struct Stage {
  u32x4 a[4];
  u32x4 w[4];     // BF16 W chunks (WQ = false) or NVFP4 codes in w[0] (WQ = true)
  uint32_t ws;    // WQ: 4 scale bytes of one W row
};

template <bool WQ>
__device__ __forceinline__ void load_stage(const Bf16Args &p, int m0, int n0, int k0, int tid,
                                           Stage<WQ> &st) {
  // A: 128 rows x 128 B = 1024 chunks of 16 B, 4 per thread
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
    int grow = m0 + row;
    grow = grow < p.M ? grow : p.M - 1;
    const int k = k0 + ch * 8;
    st.a[i] = k < p.K ? *(const u32x4 *)(p.a + (int64_t)grow * p.K + k) : u32x4{0, 0, 0, 0};
  }
  if (!WQ) {
    const uint16_t *w = (const uint16_t *)p.w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      int grow = n0 + row;
      grow = grow < p.N ? grow : p.N - 1;
      const int k = k0 + ch * 8;
      st.w[i] = k < p.K ? *(const u32x4 *)(w + (int64_t)grow * p.K + k) : u32x4{0, 0, 0, 0};
    }
  } else {
    // NVFP4: 128 rows x 32 B of codes = 256 chunks (one per thread) + 4 scale bytes per row
    const uint8_t *wq = (const uint8_t *)p.w;
    const int row = tid >> 1, half = tid & 1;
    int grow = n0 + row;
    grow = grow < p.N ? grow : p.N - 1;
    const int k = k0 + half * 32;
    st.w[0] = k < p.K ? *(const u32x4 *)(wq + (int64_t)grow * (p.K / 2) + k / 2) : u32x4{0, 0, 0, 0};
    const uint16_t *s16 = (const uint16_t *)(p.ws + (int64_t)grow * (p.K / 16) + k / 16);
    st.ws = k < p.K ? (uint32_t)s16[0] : 0u;  // 2 groups of this half-row
  }
}

template <bool WQ>
__device__ __forceinline__ void store_stage(uint8_t *la, uint8_t *lw, int tid, const Stage<WQ> &st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
    *(u32x4 *)(la + swz(row, ch)) = st.a[i];
  }
  if (!WQ) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *(u32x4 *)(lw + swz(row, ch)) = st.w[i];
    }
  } else {
    // widen 32 codes (two groups) to BF16: value = e2m1 * e4m3(scale), exact
    const int row = tid >> 1, half = tid & 1;
    const float s0 = e4m3_to_f32(st.ws & 0xFFu), s1 = e4m3_to_f32((st.ws >> 8) & 0xFFu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {      // 16 B of codes -> 4 chunks of 8 BF16
      const uint32_t word0 = st.w[0][q];
      const float s = q < 2 ? s0 : s1;  // bytes 0..7: group 0, bytes 8..15: group 1
      u32x4 out;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (word0 >> (8 * b)) & 0xFFu;
        const float lo = e2m1_to_f32(byte & 15u) * s, hi = e2m1_to_f32(byte >> 4) * s;
        out[b] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
      }
      *(u32x4 *)(lw + swz(row, half * 4 + q)) = out;
    }
  }
}

template <bool WQ>
__global__ __launch_bounds__(256, 2) void bf16_gemm_kernel(Bf16Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][BN * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int S = (p.K + BK - 1) / BK;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{0};

  Stage<WQ> st;
  load_stage<WQ>(p, m0, n0, 0, tid, st);
  store_stage<WQ>(lds_a[0], lds_w[0], tid, st);
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const int buf = s & 1;
    if (s + 1 < S) load_stage<WQ>(p, m0, n0, (s + 1) * BK, tid, st);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 fa[2], fw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *(const u32x4 *)(lds_a[buf] + swz(wm * 64 + i * 32 + l32, 2 * kk + h));
        fw[i] = *(const u32x4 *)(lds_w[buf] + swz(wn * 64 + i * 32 + l32, 2 * kk + h));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_bf16(fa[i], fw[j], acc[i][j]);
    }
    if (s + 1 < S) store_stage<WQ>(lds_a[buf ^ 1], lds_w[buf ^ 1], tid, st);
    __syncthreads();
  }

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
        const float v = WQ ? acc[i][j][r] * gs : acc[i][j][r];
        if (p.out_f32)
          ((float *)p.C)[(int64_t)row * p.N + col] = v;
        else
          ((uint16_t *)p.C)[(int64_t)row * p.N + col] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
}

}  // namespace

hipError_t launch_bf16(const Bf16Args &p, hipStream_t stream) {
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM);
  if (p.w_nvfp4)
    hipLaunchKernelGGL(bf16_gemm_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bf16_gemm_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mg
