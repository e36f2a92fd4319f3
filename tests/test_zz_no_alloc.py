"""The W4A8 entry point that allocates nothing (mgemm_w4a8_noalloc), called
through the C ABI: its output equals mgemm_w4a8's bit for bit on two calls in
a row, the second smaller (the fixed per-device buffer keeps the first call's
partials, which the second must not read), and sizes beyond the buffer are
refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def _args(inp):
    from gpu_cases import dev, scalar
    return (dev(inp["aq"]), dev(inp["atok"]), dev(inp["wq"]), dev(inp["ws"]), scalar(inp["Sw"]))


def _abi_noalloc(a, C, out_f32):
    import block_scaled_precision_tn_amd as mg
    Aq, at, Wq, Ws, Sw = a
    M, K = Aq.shape
    N = Wq.shape[0]
    rc = mg.load().mgemm_w4a8_noalloc(Aq.data_ptr(), at.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
                                      Sw.data_ptr(), C.data_ptr(), M, N, K, out_f32,
                                      torch.cuda.current_stream().cuda_stream)
    return rc


@pytest.mark.parametrize("out_f32", [1, 0])
def test_noalloc_matches_workspace_entry(out_f32):
    import block_scaled_precision_tn_amd as mg
    dt = torch.float32 if out_f32 else torch.bfloat16
    # a large call (decode kernel, 2 x 32 tokens, 28 splits; the tiled kernel
    # for 128 tokens), then a smaller one on the same buffer
    for shapes in ([(64, 5376, 14336), (8, 1000, 2048)], [(128, 1024, 8192), (1, 256, 512)]):
        for M, N, K in shapes:
            inp = synth.w4a8(M, N, K, seed=M + N)
            a = _args(inp)
            ref = torch.empty((M, N), dtype=dt, device="cuda")
            mg.mgemm_w4a8(*a, ref)
            got = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
            assert _abi_noalloc(a, got, out_f32) == 0
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                               ref.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), (M, N, K)


def test_noalloc_matches_oracle_small():
    from gpu_cases import check_f32, oracle_full, w4a8_window
    inp = synth.w4a8(33, 200, 1024, seed=5)
    C = torch.empty((33, 200), dtype=torch.float32, device="cuda")
    assert _abi_noalloc(_args(inp), C, 1) == 0
    torch.cuda.synchronize()
    c64, b64 = oracle_full("w4a8", inp)
    check_f32(C.cpu().numpy(), c64, b64, what="w4a8 noalloc", extra=w4a8_window(inp))


def test_noalloc_refuses_sizes_beyond_its_buffer():
    import block_scaled_precision_tn_amd as mg
    M, N, K = 64, 65536, 14336          # 28 splits x 64 x 65536 x 4 bytes > 48 MiB
    assert mg.mgemm_workspace_bytes(mg.OP_W4A8, M, N, K) > mg.W4A8_NOALLOC_MAX_WS
    Aq = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    at = torch.ones(M, device="cuda")
    Wq = torch.zeros((16, K // 2), dtype=torch.uint8, device="cuda")   # never read: refused first
    C = torch.zeros((1,), dtype=torch.float32, device="cuda")
    rc = mg.load().mgemm_w4a8_noalloc(Aq.data_ptr(), at.data_ptr(), Wq.data_ptr(), Wq.data_ptr(),
                                      at.data_ptr(), C.data_ptr(), M, N, K, 1,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == -4          # MGEMM_ERR_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert float(C[0]) == 0.0
