"""GPU parity of the FFN-down backward (BF16): dX = dY . W and dW = dY^T . X
against the FP64 oracle.  The oracle's operands are the same BF16 values,
arranged with numpy's transpose so that its plain sum C[m,n] = sum_k A[m,k]
W[n,k] is the gradient's definition; FP32 outputs within 1e-5 * sum |a w|,
BF16 outputs within one ulp of the oracle rounded to nearest even."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import BF16, Operand

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def _bf16(shape, std, seed, role):
    return synth.np_to_bf16_bits(synth.normal(shape, std, seed, role))


def _t(a):
    from gpu_cases import dev
    return dev(a.view(np.int16), torch.bfloat16)


def _run(kind, a, b, f32):
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import to_np
    fn = mg.mgemm_bf16_dgrad if kind == "dgrad" else mg.mgemm_bf16_wgrad
    c = fn(_t(a), _t(b), out_f32=f32)
    torch.cuda.synchronize()
    return to_np(c)


def _oracle_ops(kind, dy, b):
    # dgrad: dX[m,k] = sum_n dY[m,n] W[n,k];  wgrad: dW[n,k] = sum_m dY[m,n] X[m,k]
    if kind == "dgrad":
        return Operand(BF16, dy), Operand(BF16, np.ascontiguousarray(b.T))
    return Operand(BF16, np.ascontiguousarray(dy.T)), Operand(BF16, np.ascontiguousarray(b.T))


def _check(kind, dy, b, m=None, n=None, what=""):
    from checks import check_f32
    from gpu_cases import check_bf16_vs
    A, W = _oracle_ops(kind, dy, b)
    if m is None:
        c64, b64 = oracle.gemm_full(A, W)
    else:
        c64, b64 = oracle.gemm_points(A, W, m, n)
    g32, g16 = _run(kind, dy, b, True), _run(kind, dy, b, False)
    if m is not None:
        g32, g16 = g32[m, n], g16[m, n]
    check_f32(g32, c64, b64, what=what + " fp32")
    check_bf16_vs(g16, c64, b64, what=what + " bf16", g32=g32)


# ragged tiles in every dimension; K (and N for wgrad) multiples of 8, the
# contraction a multiple of 32
@pytest.mark.parametrize("M,N,K", [(96, 160, 264), (300, 64, 8), (1, 32, 520), (33, 96, 1000)])
def test_dgrad(M, N, K):
    dy = _bf16((M, N), 1.0, M + N, synth.ROLE_A)
    w = _bf16((N, K), 0.05, K, synth.ROLE_W)
    _check("dgrad", dy, w, what=f"dgrad {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(96, 136, 200), (32, 8, 8), (320, 264, 72), (64, 1000, 40)])
def test_wgrad(M, N, K):
    dy = _bf16((M, N), 1.0, M + N, synth.ROLE_A)
    x = _bf16((M, K), 1.0, K, synth.ROLE_W)
    _check("wgrad", dy, x, what=f"wgrad {M}x{N}x{K}")


def test_grad_repeat_bit_identical():
    dy = _bf16((128, 96), 1.0, 1, synth.ROLE_A)
    w = _bf16((96, 136), 0.05, 2, synth.ROLE_W)
    assert np.array_equal(_run("dgrad", dy, w, True), _run("dgrad", dy, w, True))
    x = _bf16((128, 136), 1.0, 3, synth.ROLE_W)
    assert np.array_equal(_run("wgrad", dy, x, True), _run("wgrad", dy, x, True))


def test_grad_full_size_sampled():
    """The FFN down projection's backward at M=4096 tokens, N=5376, K=14336."""
    M, N, K = 4096, 5376, 14336
    rng = np.random.default_rng(11)
    dy = _bf16((M, N), 1.0, 21, synth.ROLE_A)
    w = _bf16((N, K), 1.0 / np.sqrt(K), 22, synth.ROLE_W)
    m, k = rng.integers(0, M, 300), rng.integers(0, K, 300)
    _check("dgrad", dy, w, m, k, what="dgrad full")
    del w
    x = _bf16((M, K), 1.0, 23, synth.ROLE_W2)
    n, k = rng.integers(0, N, 300), rng.integers(0, K, 300)
    _check("wgrad", dy, x, n, k, what="wgrad full")
