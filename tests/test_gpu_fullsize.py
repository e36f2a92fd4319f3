"""GPU parity at the benchmark's full sizes, through the same entry points and
launch configurations that bench.py times, on outputs the oracle computes one
by one (sampled for the large GEMMs, every output for single-token decode).

Workloads are the synthetic ones bench.py uses (same generators and seeds):
  * W4A4 NVFP4 M=8192 K=14336 N=5376 (FFN down-projection shape);
  * BF16 M=4096 K=14336 N=5376;
  * W4A8 decode M in {1, 8, 32, 128}, K=14336, N=5376;
  * MXFP8 MoE GLU T=4096 H=4096 I=1536 E=64 top-8 (stage-wise on sampled
    tokens, as in test_gpu_moe).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

M, N, K = 8192, 5376, 14336


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def _points(rows, cols, n, seed):
    """n sampled output positions, always including the four corners (the
    ragged edges of the last tiles)"""
    rng = np.random.default_rng(seed)
    m = np.concatenate([[0, 0, rows - 1, rows - 1], rng.integers(0, rows, n)])
    c = np.concatenate([[0, cols - 1, 0, cols - 1], rng.integers(0, cols, n)])
    return m.astype(np.int64), c.astype(np.int64)


def test_w4a4_full_size():
    from gpu_cases import check_both, oracle_points
    inp = synth.w4a4(M, N, K, seed=0)
    m, n = _points(M, N, 300, 1)
    c64, b64 = oracle_points("w4a4", inp, m, n)
    check_both("w4a4", inp, c64, b64, m=m, n=n, what="w4a4 8192x5376x14336")


def test_bf16_full_size():
    from gpu_cases import check_both, oracle_points
    inp = synth.bf16(4096, N, K, seed=0)
    m, n = _points(4096, N, 300, 2)
    c64, b64 = oracle_points("bf16", inp, m, n)
    check_both("bf16", inp, c64, b64, m=m, n=n, what="bf16 4096x5376x14336")


@pytest.mark.parametrize("Md", [1, 8, 32, 128])
def test_w4a8_decode_full_size(Md):
    from gpu_cases import check_both, oracle_points
    inp = synth.w4a8(Md, N, K, seed=Md)
    if Md == 1:
        m, n = np.zeros(N, np.int64), np.arange(N, dtype=np.int64)   # every output
    else:
        m, n = _points(Md, N, 400, Md)
    c64, b64 = oracle_points("w4a8", inp, m, n)
    check_both("w4a8", inp, c64, b64, m=m, n=n, what=f"w4a8 decode M={Md}")


def test_moe_full_size_sampled_tokens():
    from test_gpu_moe import _check_down_combine, _check_gateup, _check_requant, run_moe
    T, H, I, E, topk = 4096, 4096, 1536, 64, 8
    inp = synth.moe(T, H, I, E, topk, seed=0)
    out, d, gu = run_moe(inp, T, H, I, E, topk, gu=True)
    tokens = np.array([0, 1, 777, 2048, 4095])
    _check_gateup(inp, gu, T, H, I, topk, tokens=tokens)
    nd = _check_requant(inp, d, T, H, I, topk, tokens=tokens)
    assert nd <= max(4, len(tokens) * topk * I // 100), nd
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


@pytest.mark.parametrize("T", [1, 16])
def test_moe_decode_full_size(T):
    """Decode-sized token counts at the full MoE shape (the swap-AB kernels)."""
    from test_gpu_moe import _check_down_combine, _check_gateup, _check_requant, run_moe
    H, I, E, topk = 4096, 1536, 64, 8
    inp = synth.moe(T, H, I, E, topk, seed=T)
    out, d, gu = run_moe(inp, T, H, I, E, topk, gu=True)
    tokens = np.arange(T) if T <= 4 else np.array([0, 5, T - 1])
    _check_gateup(inp, gu, T, H, I, topk, tokens=tokens)
    nd = _check_requant(inp, d, T, H, I, topk, tokens=tokens)
    assert nd <= max(4, len(tokens) * topk * I // 100), nd
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)
