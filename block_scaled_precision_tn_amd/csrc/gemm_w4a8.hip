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
// The operation is bound by the weight stream (N*K/2 code bytes + N*K/16
// scale bytes), so every CU must stream its share of W at full rate.  Work
// split: a workgroup owns 32 weight rows (the MFMA's B side: one lane column
// per weight row, so the per-row group scale is one value per lane) and a
// contiguous K range; its 4 waves take interleaved 32-element group pairs of
// that range and are reduced through LDS in wave order.  K ranges are split
// over `ks` workgroups (split-K); their FP32 partials go to the workspace and
// the last-arriving workgroup of each weight tile sums them in split order
// 0..ks-1, so the result is bit-identical run to run.  The tokens sit on the
// MFMA's A side (rows), padded to 32 per block; for M <= 32 only the
// accumulator registers that hold real tokens are scaled.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int NT = 32;        // weight rows per workgroup
constexpr int MAXM = 128;     // tokens per launch (larger M runs in slices)

int choose_ks(int M, int N, int K) {
  const int ntiles = (N + NT - 1) / NT;
  const int pairs = K / 32;
  const int target = M <= 32 ? 768 : 384;   // workgroups wanted in flight
  int ks = (target + ntiles - 1) / ntiles;
  ks = ks < 1 ? 1 : ks;
  ks = ks > 16 ? 16 : ks;
  while (ks > 1 && pairs / ks < 8) --ks;    // keep >= 2 pairs per wave
  return ks;
}

template <int MB, int QUADS>
__global__ __launch_bounds__(256) void w4a8_decode_kernel(W4A8Args p, int ks, float *part,
                                                          uint32_t *cnt) {
  __shared__ float red[4][MB * 16][64];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nt = blockIdx.x, kc = blockIdx.y;
  const int n = nt * NT + l32;
  const int nrow = n < p.N ? n : p.N - 1;
  const int P = p.K / 32;
  const int pbeg = (int)((int64_t)kc * P / ks), pend = (int)((int64_t)(kc + 1) * P / ks);

  f32x16 acc[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) acc[b] = f32x16{0};
  const f32x16 zero = {0};

  const uint8_t *wrow = p.wq + (int64_t)nrow * (p.K / 2);
  const uint8_t *srow = p.ws + (int64_t)nrow * (p.K / 16);


  for (int pp = pbeg + wave; pp < pend; pp += 4) {
    const u32x4 wc = *(const u32x4 *)(wrow + (int64_t)pp * 16);
    const uint32_t sb = *(const uint16_t *)(srow + (int64_t)pp * 2);
    uint64_t fa[2][MB];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const int t = b * 32 + l32;
        fa[gi][b] = t < p.M ? *(const uint64_t *)(p.aq + (int64_t)t * p.K + (2 * pp + gi) * 16 + 8 * h)
                            : (uint64_t)0;
      }
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const uint64_t fw = nvfp4x8_to_e4m3x8(wc[2 * gi + h]);
      const float s64 = e4m3_to_f32((sb >> (8 * gi)) & 0xFFu) * 64.0f;
#pragma unroll
      for (int b = 0; b < MB; ++b) {
        const f32x16 pg = mfma_fp8(e4m3x8_even_odd(fa[gi][b]), fw, zero);
#pragma unroll
        for (int r = 0; r < 4 * QUADS; ++r) acc[b][r] = __builtin_fmaf(s64, pg[r], acc[b][r]);
      }
    }
  }

  // reduce the 4 waves in wave order
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int r = 0; r < 4 * QUADS; ++r) red[wave][b * 16 + r][lane] = acc[b][r];
  __syncthreads();

  const float sw = *p.Sw;
  if (ks == 1) {
    if (wave == 0 && n < p.N) {
#pragma unroll
      for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int r = 0; r < 4 * QUADS; ++r) {
          const int t = b * 32 + acc_row(r, lane);
          if (t >= p.M) continue;
          const int q = b * 16 + r;
          const float v = (((red[0][q][lane] + red[1][q][lane]) + red[2][q][lane]) + red[3][q][lane]) *
                          (p.atok[t] * sw);
          if (p.out_f32)
            ((float *)p.C)[(int64_t)t * p.N + n] = v;
          else
            ((uint16_t *)p.C)[(int64_t)t * p.N + n] = (uint16_t)f32_to_bf16_rne(v);
        }
    }
    return;
  }

  // split-K: publish this split's partial, the last arrival reduces in order
  if (wave == 0 && n < p.N) {
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
      for (int r = 0; r < 4 * QUADS; ++r) {
        const int t = b * 32 + acc_row(r, lane);
        if (t >= p.M) continue;
        const int q = b * 16 + r;
        part[((int64_t)kc * p.M + t) * p.N + n] =
            ((red[0][q][lane] + red[1][q][lane]) + red[2][q][lane]) + red[3][q][lane];
      }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&cnt[nt], 1u) == (uint32_t)(ks - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = tid; e < p.M * NT; e += 256) {
    const int t = e / NT, nn = nt * NT + (e % NT);
    if (nn >= p.N) continue;
    float v = 0.0f;
    for (int s = 0; s < ks; ++s) v += part[((int64_t)s * p.M + t) * p.N + nn];
    v *= p.atok[t] * sw;
    if (p.out_f32)
      ((float *)p.C)[(int64_t)t * p.N + nn] = v;
    else
      ((uint16_t *)p.C)[(int64_t)t * p.N + nn] = (uint16_t)f32_to_bf16_rne(v);
  }
  if (tid == 0) atomicExch(&cnt[nt], 0u);  // leave the counter ready for the next call
}

template <int MB, int QUADS>
void launch_one(const W4A8Args &p, int ks, float *part, uint32_t *cnt, hipStream_t stream) {
  dim3 grid((p.N + NT - 1) / NT, ks);
  hipLaunchKernelGGL((w4a8_decode_kernel<MB, QUADS>), grid, dim3(256), 0, stream, p, ks, part, cnt);
}

// Workspace: a fixed 64 KiB counter region first (one counter per 32-row
// weight tile; left at zero by every call), then the split partials.  The
// fixed placement keeps the counters away from partials of any earlier call.
constexpr size_t kCounterBytes = 65536;

}  // namespace

size_t w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t Ms = M < MAXM ? M : MAXM;
  const int ks = choose_ks((int)Ms, (int)N, (int)K);
  if (ks <= 1) return 0;
  return kCounterBytes + (size_t)ks * (size_t)Ms * (size_t)N * sizeof(float);
}

int64_t w4a8_max_n() { return (int64_t)(kCounterBytes / sizeof(uint32_t)) * NT; }

hipError_t launch_w4a8(const W4A8Args &p0, hipStream_t stream) {
  for (int m0 = 0; m0 < p0.M; m0 += MAXM) {
    W4A8Args p = p0;
    p.M = p0.M - m0 < MAXM ? p0.M - m0 : MAXM;
    p.aq = p0.aq + (int64_t)m0 * p0.K;
    p.atok = p0.atok + m0;
    p.C = (char *)p0.C + (int64_t)m0 * p0.N * (p0.out_f32 ? 4 : 2);
    const int Mslice = p0.M < MAXM ? p0.M : MAXM;
    const int ks = choose_ks(Mslice, p.N, p.K);
    float *part = nullptr;
    uint32_t *cnt = nullptr;
    if (ks > 1) {
      cnt = (uint32_t *)p0.work;
      part = (float *)((char *)p0.work + kCounterBytes);
    }
    if (p.M > 96) launch_one<4, 4>(p, ks, part, cnt, stream);
    else if (p.M > 64) launch_one<3, 4>(p, ks, part, cnt, stream);
    else if (p.M > 32) launch_one<2, 4>(p, ks, part, cnt, stream);
    else if (p.M > 24) launch_one<1, 4>(p, ks, part, cnt, stream);
    else if (p.M > 16) launch_one<1, 3>(p, ks, part, cnt, stream);
    else if (p.M > 8) launch_one<1, 2>(p, ks, part, cnt, stream);
    else launch_one<1, 1>(p, ks, part, cnt, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mg
