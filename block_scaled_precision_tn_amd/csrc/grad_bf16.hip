// grad_bf16.hip -- backward of the BF16 FFN down projection y = x . W^T (the
// H3 FFN-down operator of RL-Kernel PR #535 and its gradients):
//   input gradient  dX[M,K] = dY[M,N] . W[N,K]      (contraction over N)
//   weight gradient dW[N,K] = dY[M,N]^T . X[M,K]    (contraction over M)
// Neither contraction runs along the stored rows of every operand, so each
// gradient first writes the operands it needs contraction-major into the
// workspace with an LDS-tiled transpose (an HBM-bound copy: 0.15 GB for W,
// 0.16 GB for dY and X at the FFN-down shape, against a 0.63 TFLOP GEMM) and
// then runs the TN BF16 GEMM kernel, whose every output sums its contraction
// in one fixed order: results are run-to-run bit-identical.
#include "common.h"
#include "kernels.h"

namespace mg {
namespace {

constexpr int TT = 64;          // transpose tile
constexpr int TP = TT + 2;      // LDS pitch (elements): rows start in distinct banks

// out[C,R] = in[R,C]^T (BF16), C % 8 == 0 and R % 8 == 0
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t *in, uint16_t *out, int R,
                                                        int C) {
  __shared__ uint16_t t[TT * TP];
  const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT, tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // 64 rows x 8 chunks of 8 elements
    const int q = tid + 256 * i, row = q >> 3, c8 = q & 7;
    const int r = r0 + row, c = c0 + 8 * c8;
    u32x4 v = {0, 0, 0, 0};
    if (r < R && c < C) v = *(const u32x4 *)(in + (int64_t)r * C + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[row * TP + 8 * c8 + 2 * j] = (uint16_t)(v[j] & 0xFFFFu);
      t[row * TP + 8 * c8 + 2 * j + 1] = (uint16_t)(v[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {   // 64 output rows (input columns) x 8 chunks
    const int q = tid + 256 * i, col = q >> 3, r8 = q & 7;
    const int c = c0 + col, r = r0 + 8 * r8;
    if (c >= C || r >= R) continue;
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = (uint32_t)t[(8 * r8 + 2 * j) * TP + col] | ((uint32_t)t[(8 * r8 + 2 * j + 1) * TP + col] << 16);
    *(u32x4 *)(out + (int64_t)c * R + r) = v;
  }
}

hipError_t transpose(const uint16_t *in, uint16_t *out, int R, int C, hipStream_t stream) {
  hipLaunchKernelGGL(k_transpose_bf16, dim3((C + TT - 1) / TT, (R + TT - 1) / TT), dim3(256), 0,
                     stream, in, out, R, C);
  return hipGetLastError();
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// transposed operands, then the TN product's tail partials (bf16_workspace_bytes)
size_t bf16_grad_workspace_bytes(bool wgrad, int64_t M, int64_t N, int64_t K) {
  if (!wgrad) return up256((size_t)N * (size_t)K * 2) + bf16_workspace_bytes(M, K, N);
  return up256((size_t)M * (size_t)N * 2) + up256((size_t)M * (size_t)K * 2) +
         bf16_workspace_bytes(N, K, M);
}

hipError_t launch_bf16_dgrad(const uint16_t *dY, const uint16_t *W, void *dX, int M, int N, int K,
                             int out_f32, void *ws, hipStream_t stream) {
  uint16_t *wt = (uint16_t *)ws;                 // W^T [K,N]
  hipError_t e = transpose(W, wt, N, K, stream);
  if (e != hipSuccess) return e;
  Bf16Args p{dY, wt, nullptr, nullptr, dX, M, K, N, out_f32, 0};
  return launch_bf16(p, (char *)ws + up256((size_t)N * (size_t)K * 2), stream);
}

hipError_t launch_bf16_wgrad(const uint16_t *dY, const uint16_t *X, void *dW, int M, int N, int K,
                             int out_f32, void *ws, hipStream_t stream) {
  uint16_t *dyt = (uint16_t *)ws;                                         // dY^T [N,M]
  uint16_t *xt = (uint16_t *)((char *)ws + up256((size_t)M * (size_t)N * 2));  // X^T [K,M]
  hipError_t e = transpose(dY, dyt, M, N, stream);
  if (e != hipSuccess) return e;
  e = transpose(X, xt, M, K, stream);
  if (e != hipSuccess) return e;
  Bf16Args p{dyt, xt, nullptr, nullptr, dW, N, K, M, out_f32, 0};
  return launch_bf16(p, (char *)xt + up256((size_t)M * (size_t)K * 2), stream);
}

}  // namespace mg
