"""GPU parity of the small-M W4A16 path (up to 128 tokens: the decode kernel
that streams NVFP4 weights, widens them to BF16 in registers and splits K
over workgroups) against the FP64 oracle, through the C ABI.

Shapes cover one, two and four 32-token blocks (65 to 128 tokens: one
launch on 128-row weight tiles), the switch to the tiled kernel above 128
tokens, partial last K ranges, K/16 not a multiple of 16, N not a multiple
of the 64- or 128-row tile, and a K that fits one range (no split).  The
full-size cases are the workload the bench times: K = 14336, N = 5376,
M in {1, 16, 128}.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def test_w4a16_identity_decode_probe():
    """A = identity rows (BF16 1.0), S_w = 1: the FP32 output is each weight
    element e2m1 * e4m3 exactly, for every code byte and every non-NaN scale
    byte (negative and subnormal ones included), through each of the decode
    kernel's widening forms (1 token, up to 8, up to 16, up to 64, up to 128
    tokens), so the in-register widening and its K order are bit-exact."""
    from gpu_cases import gpu_w4a16
    rng = np.random.default_rng(21)
    N, K = 200, 256
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0, 256, (N, K // 16), dtype=np.uint8)
    ws[(ws & 0x7F) == 0x7F] -= 1                          # no NaN bytes here
    ws.reshape(-1)[:254] = [b for b in range(256) if b & 0x7F != 0x7F]   # every other byte
    ident = np.zeros((K, K), np.uint16)
    np.fill_diagonal(ident, 0x3F80)
    ref = oracle.elem_values(oracle.Operand(oracle.NVFP4, wq, ws)).T
    for M in (1, 2, 8, 9, 16, 17, 32, 33, 64, 128):
        c = gpu_w4a16(dict(a=ident[:M].copy(), wq=wq, ws=ws, Sw=1.0), True)
        assert np.array_equal(c.astype(np.float64), ref[:M]), M


@pytest.mark.parametrize("M", [1, 5, 16, 40, 129])
def test_w4a16_nan_scale_propagates(M):
    """A NaN group scale (E4M3 byte 0x7F) makes every output of its weight row
    NaN, as in the oracle; all other outputs stay finite and within tolerance."""
    from gpu_cases import gpu_w4a16, oracle_full
    from checks import check_f32
    inp = synth.w4a16(M, 130, 1024, seed=M)
    inp["ws"][7, 20] = 0x7F
    c = gpu_w4a16(inp, True)
    c64, b64 = oracle_full("w4a16", inp)
    assert np.array_equal(np.isnan(c), np.isnan(c64))
    assert np.isnan(c[:, 7]).all() and not np.isnan(np.delete(c, 7, axis=1)).any()
    check_f32(np.delete(c, 7, axis=1), np.delete(c64, 7, axis=1), np.delete(b64, 7, axis=1))


@pytest.mark.parametrize("M", [1, 3, 16, 32, 33, 64, 65, 100, 128, 129])
@pytest.mark.parametrize("N,K", [(96, 256), (200, 1024),
                                 (130, 1536),    # three 512-element K ranges
                                 (257, 1568),    # partial last range, K/16 not a multiple of 16
                                 (96, 64)])      # one range: no split
def test_w4a16_small_m_parity(M, N, K):
    from gpu_cases import check_both, oracle_full
    inp = synth.w4a16(M, N, K, seed=M + 7 * N)
    c64, b64 = oracle_full("w4a16", inp)
    check_both("w4a16", inp, c64, b64, what=f"w4a16 {M}x{N}x{K}")


def test_w4a16_small_m_repeat_bit_identical():
    from gpu_cases import gpu_w4a16
    inp = synth.w4a16(48, 320, 2048, seed=3)
    c1 = gpu_w4a16(inp, True)
    c2 = gpu_w4a16(inp, True)
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))


def test_w4a16_small_m_workspace_reuse_and_refusal():
    """An explicit workspace of exactly the reported size, with arbitrary
    contents, works twice in a row; one byte less is refused before any work
    is enqueued."""
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import dev, out_tensor, scalar, to_np, oracle_full, check_f32
    M, N, K = 16, 192, 1024
    inp = synth.w4a16(M, N, K, seed=9)
    need = mg.mgemm_workspace_bytes(mg.OP_W4A16, M, N, K)
    assert need == M * N * 4   # one 1024-element K range
    A = dev(inp["a"].view(np.int16), torch.bfloat16)
    args = (A, dev(inp["wq"]), dev(inp["ws"]), scalar(inp["Sw"]))
    C = out_tensor(M, N, True)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    c64, b64 = oracle_full("w4a16", inp)
    for _ in range(2):
        mg.mgemm_w4a16(*args, C, ws=ws)
        torch.cuda.synchronize()
        check_f32(to_np(C), c64, b64)
    with pytest.raises(ValueError):
        mg.mgemm_w4a16(*args, C, ws=ws[:need - 1])


@pytest.mark.parametrize("Md", [1, 16, 128])
def test_w4a16_decode_full_size(Md):
    from gpu_cases import check_both, oracle_points
    N, K = 5376, 14336
    inp = synth.w4a16(Md, N, K, seed=Md)
    if Md == 1:
        m, n = np.zeros(N, np.int64), np.arange(N, dtype=np.int64)   # every output
    else:
        rng = np.random.default_rng(Md)
        m = np.concatenate([[0, 0, Md - 1, Md - 1], rng.integers(0, Md, 400)]).astype(np.int64)
        n = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 400)]).astype(np.int64)
    c64, b64 = oracle_points("w4a16", inp, m, n)
    check_both("w4a16", inp, c64, b64, m=m, n=n, what=f"w4a16 decode M={Md}")
