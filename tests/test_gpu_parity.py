"""GPU parity: every entry point of the HIP library against the FP64 oracle.

Sizes here span several workgroup tiles plus ragged M/N tails and K tails,
and the oracle computes every output.  Full-size workloads (sampled outputs)
are in test_gpu_fullsize.py.  All calls go through the C ABI via the Python
binding; nothing here falls back to a CPU path.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from checks import check_f32

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()  # must exist: no fallback
    yield


def _hex(rows):
    return np.array([[int(x, 16) for x in r] for r in rows], dtype=np.uint8)


# ----------------------------------------------------------- hand cases
HAND = json.load(open(os.path.join(GOLD, "hand_cases.json")))["cases"]


def _hand_inputs(c):
    if c["fmt"] == "w4a4":
        return "w4a4", dict(aq=_hex(c["aq"]), as_=_hex(c["as"]), Sa=c["Sa"], wq=_hex(c["wq"]),
                            ws=_hex(c["ws"]), Sw=c["Sw"])
    if c["fmt"] == "w4a8":
        return "w4a8", dict(aq=_hex(c["a8"]), atok=np.array(c["atok"], np.float32),
                            wq=_hex(c["wq"]), ws=_hex(c["ws"]), Sw=c["Sw"])
    if c["fmt"] == "w4a16":
        a = np.array([[int(x, 16) for x in r] for r in c["a16"]], dtype=np.uint16)
        return "w4a16", dict(a=a, wq=_hex(c["wq"]), ws=_hex(c["ws"]), Sw=c["Sw"])
    return None, None


def _pad_k(fmt, inp, K):
    """The library needs K % 32 == 0: extend a K = 16 case with zero elements
    (zero codes under scale 1.0), which leaves every product unchanged."""
    if K % 32 == 0:
        return inp
    out = dict(inp)
    pad = lambda a, v=0: np.pad(a, ((0, 0), (0, a.shape[1])), constant_values=v)  # noqa: E731
    out["wq"], out["ws"] = pad(inp["wq"]), pad(inp["ws"], 0x38)
    if fmt == "w4a4":
        out["aq"], out["as_"] = pad(inp["aq"]), pad(inp["as_"], 0x38)
    elif fmt == "w4a8":
        out["aq"] = pad(inp["aq"])
    else:
        out["a"] = pad(inp["a"])
    return out


@pytest.mark.parametrize("case", [c for c in HAND if c["fmt"] != "mxfp8"], ids=lambda c: c["name"])
def test_hand_cases_bit_exact(case):
    from gpu_cases import GPU
    fmt, inp = _hand_inputs(case)
    inp = _pad_k(fmt, inp, case["K"])
    c32 = GPU[fmt](inp, True)
    assert np.array_equal(c32.astype(np.float64), np.array(case["C"])), c32
    c16 = GPU[fmt](inp, False)
    assert np.array_equal(c16, np.array([[int(x, 16) for x in r] for r in case["bf16"]], np.uint16))


# ------------------------------------------------------ decode probe (P6)
def test_w4a4_identity_decode_probe():
    """W = identity (code 2 = 1.0, scale 0x38, S_w = 1): FP32 C equals the
    decoded activations exactly, so every code x scale decode is bit-exact."""
    from gpu_cases import gpu_w4a4
    rng = np.random.default_rng(11)
    M, K = 64, 256
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)
    codes = np.zeros((K, K), np.uint8)
    np.fill_diagonal(codes, 2)
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.full((K, K // 16), 0x38, np.uint8)
    c = gpu_w4a4(dict(aq=aq, as_=as_, Sa=1.0, wq=wq, ws=ws, Sw=1.0), True)
    ref = oracle.elem_values(oracle.Operand(oracle.NVFP4, aq, as_))
    assert np.array_equal(c.astype(np.float64), ref)
    # the same probe with the roles swapped decodes the weight side
    c = gpu_w4a4(dict(aq=wq, as_=ws, Sa=1.0, wq=aq, ws=as_, Sw=1.0), True)
    assert np.array_equal(c.astype(np.float64), ref.T)


def test_w4a8_identity_decode_probe():
    from gpu_cases import gpu_w4a8
    rng = np.random.default_rng(12)
    N, K = 96, 128
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    a8 = np.zeros((K, K), np.uint8)
    np.fill_diagonal(a8, 0x38)  # E4M3 1.0
    for M in (1, 8, 32, 128):
        c = gpu_w4a8(dict(aq=a8[:M].copy(), atok=np.ones(M, np.float32), wq=wq, ws=ws, Sw=1.0), True)
        ref = oracle.elem_values(oracle.Operand(oracle.NVFP4, wq, ws)).T[:M]
        assert np.array_equal(c.astype(np.float64), ref), M


# -------------------------------------------------------- random parity
def _w4a4_inputs(M, N, K, seed):
    d = synth.w4a4(M, N, K, seed=seed)
    return d


SHAPES = [(1, 32, 32), (130, 200, 544), (256, 384, 1024), (77, 129, 96)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a4_parity(M, N, K):
    from gpu_cases import check_both, oracle_full
    inp = _w4a4_inputs(M, N, K, seed=M + N + K)
    c64, b64 = oracle_full("w4a4", inp)
    check_both("w4a4", inp, c64, b64, what=f"w4a4 {M}x{N}x{K}")


# Large W4A4 calls take a 256 x 256 or a 256 x 224 tile, whichever fills the
# device's rounds with less work (256 CUs: 4096 x 4096 takes 256 x 256, one
# round against two; 1000-wide N and 8192 x 5376 take 256 x 224).  Both are
# bit-exact against the route emulation at sampled outputs (corners included).
@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (520, 1000, 544), (1024, 5376, 512)])
def test_w4a4_tile_widths(M, N, K):
    from gpu_cases import check_both, oracle_points
    inp = _w4a4_inputs(M, N, K, seed=M + N)
    rng = np.random.default_rng(M)
    m = np.concatenate([[0, 0, M - 1, M - 1, 255, 256], rng.integers(0, M, 400)]).astype(np.int64)
    n = np.concatenate([[0, N - 1, 0, N - 1, 223, 224], rng.integers(0, N, 400)]).astype(np.int64)
    c64, b64 = oracle_points("w4a4", inp, m, n)
    check_both("w4a4", inp, c64, b64, m=m, n=n, what=f"w4a4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_parity(M, N, K):
    from gpu_cases import check_both, oracle_full
    inp = synth.bf16(M, N, K, seed=M * 3 + K)
    c64, b64 = oracle_full("bf16", inp)
    check_both("bf16", inp, c64, b64, what=f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SHAPES + [(16, 256, 512)])
def test_w4a16_parity(M, N, K):
    from gpu_cases import check_both, oracle_full
    inp = synth.w4a16(M, N, K, seed=0 if (M, N, K) == (16, 256, 512) else M + 5)
    c64, b64 = oracle_full("w4a16", inp)
    check_both("w4a16", inp, c64, b64, what=f"w4a16 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 3, 8, 17, 32, 33, 100, 128, 200])
@pytest.mark.parametrize("N,K", [(96, 256), (200, 1024), (384, 2048),
                                 (130, 1536),    # odd number of 512-element K ranges
                                 (257, 1568),    # partial last range, K/16 not a multiple of 16
                                 (96, 64)])      # one stage of K: no split (tiled path for M > 64)
def test_w4a8_parity(M, N, K):
    from gpu_cases import check_both, oracle_full
    inp = synth.w4a8(M, N, K, seed=M + N)
    c64, b64 = oracle_full("w4a8", inp)
    check_both("w4a8", inp, c64, b64, what=f"w4a8 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 40])
def test_w4a8_parity_long_k(M):
    """K = 16896 gives 33 split-K partials, one more than the reduction
    requests up front: the rest of the sum takes its tail loop."""
    from gpu_cases import check_both, oracle_full
    N, K = 96, 16896
    inp = synth.w4a8(M, N, K, seed=M + 3)
    c64, b64 = oracle_full("w4a8", inp)
    check_both("w4a8", inp, c64, b64, what=f"w4a8 {M}x{N}x{K}")


def test_w4a8_workspace_reuse_across_sizes():
    """One workspace serves a large call then smaller ones (the split-K
    partials it holds need no clearing between calls)."""
    from gpu_cases import check_both, oracle_full
    for M, N, K in [(128, 384, 2048), (8, 200, 1024), (32, 384, 2048), (1, 96, 256)]:
        inp = synth.w4a8(M, N, K, seed=7 * M + 1)
        c64, b64 = oracle_full("w4a8", inp)
        check_both("w4a8", inp, c64, b64, what=f"w4a8 reuse {M}x{N}x{K}")


# ----------------------------------------------------------- invariants
def test_repeat_bit_identical_and_chunked_rows():
    """Same call twice is bit-identical; splitting M into two calls stays within
    tolerance (RL-Kernel PR #535 checks repeat and chunked invariance)."""
    from gpu_cases import GPU, oracle_full
    inp = synth.w4a4(192, 256, 512, seed=21)
    a = GPU["w4a4"](inp, True)
    b = GPU["w4a4"](inp, True)
    assert np.array_equal(a, b)
    top = {k: (v[:100] if k in ("aq", "as_") else v) for k, v in inp.items()}
    bot = {k: (v[100:] if k in ("aq", "as_") else v) for k, v in inp.items()}
    c = np.concatenate([GPU["w4a4"](top, True), GPU["w4a4"](bot, True)])
    c64, b64 = oracle_full("w4a4", inp)
    check_f32(c, c64, b64, what="chunked")
    inp8 = synth.w4a8(32, 384, 2048, seed=22)
    assert np.array_equal(GPU["w4a8"](inp8, True), GPU["w4a8"](inp8, True))
    inpb = synth.bf16(128, 256, 512, seed=23)
    assert np.array_equal(GPU["bf16"](inpb, False), GPU["bf16"](inpb, False))


def test_sign_and_scale_invariants():
    """Flipping the sign bits of weight row n negates column n bit-exactly;
    raising its E4M3 scale exponents by one doubles it bit-exactly."""
    from gpu_cases import GPU
    inp = synth.w4a4(64, 96, 256, seed=31)
    c0 = GPU["w4a4"](inp, True)
    wq = inp["wq"].copy()
    wq[5] ^= 0x88
    c1 = GPU["w4a4"](dict(inp, wq=wq), True)
    assert np.array_equal(c1[:, 5], -c0[:, 5])
    ws = inp["ws"].copy()
    ok = (ws[7] & 0x78) < 0x70
    ws[7] = np.where(ok, ws[7] + 8, ws[7])
    if ok.all():
        c2 = GPU["w4a4"](dict(inp, ws=ws), True)
        assert np.array_equal(c2[:, 7], 2 * c0[:, 7])


def test_nan_scale_propagates():
    """An E4M3 NaN scale byte (0x7F or 0xFF) makes every output that reads its
    group NaN, as in the oracle's decode; all other outputs are unchanged
    bit for bit (W4A4, FP32 output)."""
    from gpu_cases import GPU, oracle_full
    inp = synth.w4a4(64, 96, 256, seed=41)
    c0 = GPU["w4a4"](inp, True)
    as_ = inp["as_"].copy()
    as_[3, 5] = 0x7F
    ws = inp["ws"].copy()
    ws[10, 2] = 0xFF
    bad = dict(inp, as_=as_, ws=ws)
    c1 = GPU["w4a4"](bad, True)
    nan = np.zeros(c1.shape, bool)
    nan[3, :] = True
    nan[:, 10] = True
    c64, _ = oracle_full("w4a4", bad)
    assert np.array_equal(np.isnan(c64), nan)
    assert np.array_equal(np.isnan(c1), nan)
    assert np.array_equal(c1[~nan], c0[~nan])


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 256), (520, 1000, 544)])
def test_nan_scale_propagates_wide_tiles(M, N, K):
    """The same on the 256 x 256 and 256 x 224 tiles, whose scale operands
    carry a stage's four group scale bytes at once: NaN bytes in the first
    and last group of a row or column make exactly that row or column NaN
    (as the oracle's decode does for any group), the rest stays bit for bit."""
    from gpu_cases import GPU
    inp = synth.w4a4(M, N, K, seed=43)
    G = K // 16
    c0 = GPU["w4a4"](inp, True)
    as_ = inp["as_"].copy()
    as_[3, 5] = 0x7F
    as_[M - 2, G - 1] = 0xFF
    ws = inp["ws"].copy()
    ws[10, 2] = 0xFF
    ws[N - 1, 0] = 0x7F
    c1 = GPU["w4a4"](dict(inp, as_=as_, ws=ws), True)
    nan = np.zeros(c1.shape, bool)
    nan[[3, M - 2], :] = True
    nan[:, [10, N - 1]] = True
    assert np.array_equal(np.isnan(c1), nan)
    assert np.array_equal(c1[~nan], c0[~nan])


# ------------------------------------------------------------------- plan
def test_plan_on_device():
    import block_scaled_precision_tn_amd as mg
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch
    assert mg.mgemm_plan(0, mg.FMT_NVFP4, mg.FMT_NVFP4) == (mg.EXEC_FP8_EXACT, mg.MMA_FP8, 3)
    assert mg.mgemm_plan(0, mg.FMT_NVFP4, mg.FMT_FP8_E4M3_TOKEN) == (mg.EXEC_FP8_EXACT, mg.MMA_FP8, 4)
    assert mg.mgemm_plan(0, mg.FMT_BF16, mg.FMT_BF16)[0] == mg.EXEC_NATIVE
    # a pair with no path is refused, never re-run at a wider format
    with pytest.raises(mg.MgemmError) as ei:
        A = torch.zeros((32, 32), dtype=torch.uint8, device="cuda")
        mg.load().mgemm_bf16  # exists
        rc = mg.load().mgemm_w4a16(A.data_ptr(), A.data_ptr(), A.data_ptr(), A.data_ptr(),
                                   A.data_ptr(), 32, 32, 33, 0, None, 0, None)
        mg._check("mgemm_w4a16", rc)
    assert ei.value.status == -2


def test_w4a8_concurrent_streams_own_workspaces():
    """Calls on two streams get two cached workspaces (their split-K partials
    never mix) and both results match the oracle."""
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import check_f32, dev, oracle_full, scalar
    cur = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    runs = []
    for s, seed in ((s1, 61), (s2, 62)):
        inp = synth.w4a8(16, 384, 2048, seed=seed)
        args = (dev(inp["aq"]), dev(inp["atok"]), dev(inp["wq"]), dev(inp["ws"]), scalar(inp["Sw"]))
        runs.append((s, inp, args, torch.empty((16, 384), dtype=torch.float32, device="cuda")))
    for s, _, _, _ in runs:
        s.wait_stream(cur)                      # inputs were copied on the current stream
    for _ in range(3):
        for s, _, args, C in runs:
            mg.mgemm_w4a8(*args, C, stream=s)
    torch.cuda.synchronize()
    w1 = mg.workspace(1, "w4a8", s1)
    w2 = mg.workspace(1, "w4a8", s2)
    assert w1.data_ptr() != w2.data_ptr()
    for _, inp, _, C in runs:
        c64, b64 = oracle_full("w4a8", inp)
        from gpu_cases import w4a8_window
        check_f32(C.cpu().numpy(), c64, b64, what="w4a8 stream", extra=w4a8_window(inp))


@pytest.mark.parametrize("M,N,K", [(300, 640, 2048),    # 6 tiles of 256 x 256, all split (8 ranges)
                                   (520, 1000, 1568),   # partial K stage in the last range
                                   (300, 652, 2048),    # N % 8 != 0: the sum's element-wise stores
                                   (256, 384, 1024)])
def test_bf16_tail_split(M, N, K):
    """Grids that leave a partial last round split those tiles along K (FP32
    partial tiles, then an ordered sum): parity with the oracle in FP32 and
    BF16, repeat bit-identical, an explicit workspace of exactly the reported
    size with arbitrary contents accepted, one byte less refused."""
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import check_both, oracle_full, dev, out_tensor, to_np
    inp = synth.bf16(M, N, K, seed=M + N)
    c64, b64 = oracle_full("bf16", inp)
    check_both("bf16", inp, c64, b64, what=f"bf16 split {M}x{N}x{K}")
    need = mg.mgemm_workspace_bytes(mg.OP_BF16, M, N, K)
    assert need > 0
    A = dev(inp["a"].view(np.int16), torch.bfloat16)
    W = dev(inp["w"].view(np.int16), torch.bfloat16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        C = out_tensor(M, N, True)
        mg.mgemm_bf16(A, W, C, ws=ws)
        torch.cuda.synchronize()
        outs.append(to_np(C))
    check_f32(outs[0], c64, b64)
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    with pytest.raises(ValueError):
        mg.mgemm_bf16(A, W, out_tensor(M, N, True), ws=ws[:need - 1])


@pytest.mark.parametrize("M,N,K", [(4000, 4000, 96),    # 256 ragged tiles: one whole round
                                   (4000, 4100, 512)])  # 272 tiles: 256 whole, 16 split in 2
def test_bf16_whole_tiles(M, N, K):
    """Grids of at least one tile per CU: whole tiles (the partial K stage
    included) next to split ones, every output against the oracle."""
    from gpu_cases import check_both, oracle_full
    inp = synth.bf16(M, N, K, seed=M + K)
    c64, b64 = oracle_full("bf16", inp)
    check_both("bf16", inp, c64, b64, what=f"bf16 whole tiles {M}x{N}x{K}")
