"""GPU parity of the NVFP4 grouped MoE GLU against the FP64 oracle.

As for the MXFP8 MoE, the in-path re-quantisation of h is a decision point,
so parity is stage-wise:
  (ii)  the kernel's NVFP4 h (debug tap) equals the oracle's, except where the
        oracle's h (or a group's amax / 6 / Sh) lies within the FP32
        accumulation bound of a rounding boundary: there every GPU code must
        still be a correct rounding of some h' within that bound;
  (iii) the kernel's output equals the oracle's down projection and combine
        applied to the kernel's own h: FP32 tolerance / 1 BF16 ulp.
Both GEMMs run on the exact FP8 route: each group term is exact in FP32, so
the accumulation tolerance is 1e-5 * sum |a w| with no FP8 window term.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def run_moe4(inp, T, H, I, E, topk):
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import dev
    f32 = lambda v: torch.tensor(np.atleast_1d(np.asarray(v, np.float32)), device="cuda")  # noqa: E731
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dbg = torch.zeros(T * topk * (I // 2 + I // 16), dtype=torch.uint8, device="cuda")
    mg.mgemm_moe_nvfp4_glu(dev(inp["xq"]), dev(inp["xs"]), f32(inp["Sx"]), dev(inp["ids"]),
                           dev(inp["tw"]), dev(inp["w13q"]), dev(inp["w13s"]), f32(inp["Sw13"]),
                           dev(inp["w2q"]), dev(inp["w2s"]), f32(inp["Sw2"]), f32(inp["Sh"]),
                           out, dbg_h=dbg)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return o, dbg.cpu().numpy().reshape(T * topk, I // 2 + I // 16)


def _e4m3(b):
    return torch.tensor(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _unpack(q):
    return np.stack([q & 15, q >> 4], axis=-1).reshape(-1)


def _check_requant(inp, d, T, H, I, topk, tokens, tol=1e-5):
    """Stage (ii); returns the number of codes that differ from the oracle's."""
    from scipy.special import expit
    Sh = float(inp["Sh"])
    n_diff = 0
    for t in tokens:
        for j in range(topk):
            e = int(inp["ids"][t, j])
            if not 0 <= e < inp["w13q"].shape[0]:
                continue                         # a dropped slot
            g, u, bg, bu = oracle.moe4_gateup(inp, t, e, H, I)
            hq, hs = oracle.moe4_glu_requant(g, u, Sh)
            gq, gs = d[t * topk + j, :I // 2], d[t * topk + j, I // 2:]
            if np.array_equal(hq, gq) and np.array_equal(hs, gs):
                continue
            s = expit(g)
            h = g * s * u
            dh = np.abs(s * (1 + g * (1 - s)) * u) * tol * bg + np.abs(g * s) * tol * bu + \
                4 * 2.0 ** -24 * np.abs(h)
            oc, gc = _unpack(hq), _unpack(gq)
            for b in range(I // 16):
                sl = slice(16 * b, 16 * b + 16)
                amax, damax = np.max(np.abs(h[sl])), np.max(dh[sl])
                if hs[b] != gs[b]:
                    # the scale bytes differ by one step, where amax / 6 / Sh
                    # lies within its bound of the midpoint of the two values
                    assert abs(int(hs[b]) - int(gs[b])) == 1, (t, j, b, hs[b], gs[b])
                    mid = (_e4m3(hs[b]) + _e4m3(gs[b])) / 2
                    assert abs(amax / 6 / Sh - mid) <= 2 * damax / 6 / Sh + 2.0 ** -20 * mid, \
                        (t, j, b, amax, hs[b], gs[b])
                dsc = float(_e4m3(gs[b])) * Sh
                if dsc == 0:
                    assert not gc[sl].any()
                    continue
                x, tx = h[sl] / dsc, 2 * dh[sl] / dsc + 2.0 ** -20
                c = gc[sl]
                m = GRID[c & 7]
                lo = np.where(c & 7, (m + GRID[np.maximum((c & 7) - 1, 0)]) / 2, 0.0)
                hi = np.where((c & 7) < 7, (m + GRID[np.minimum((c & 7) + 1, 7)]) / 2, np.inf)
                ax = np.abs(x)
                ok = (ax >= lo - tx) & (ax <= hi + tx)
                ok &= (np.sign(x) == np.where(c & 8, -1, 1)) | (m == 0) | (ax <= tx)
                assert ok.all(), (t, j, b, np.where(~ok)[0], x[~ok], c[~ok])
                n_diff += int((gc[sl] != oc[sl]).sum())
    return n_diff


def _check_down_combine(inp, d, out, T, H, I, topk, tokens):
    """Stage (iii): oracle down projection + combine on the GPU's h."""
    from gpu_cases import check_bf16_vs
    Sh = float(inp["Sh"])
    ref = np.zeros((len(tokens), H))
    bnd = np.zeros((len(tokens), H))
    for ti, t in enumerate(tokens):
        for j in range(topk):
            e = int(inp["ids"][t, j])
            if not 0 <= e < inp["w13q"].shape[0]:
                continue                         # a dropped slot
            row = d[t * topk + j]
            y, by = oracle.moe4_down(row[:I // 2].copy(), row[I // 2:].copy(), Sh, e, inp, H, I)
            w = float(inp["tw"][t, j])
            ref[ti] += w * y
            bnd[ti] += abs(w) * by
    extra = topk * 2.0 ** -23 * bnd
    check_bf16_vs(out[tokens], ref, bnd, what="moe4 out", extra=extra)


def test_moe4_hand_case():
    g = json.load(open(os.path.join(GOLD, "moe_nvfp4_hand.json")))
    H, I = g["H"], g["I"]
    b = lambda k: int(g[k], 16)  # noqa: E731
    inp = dict(xq=np.full((1, H // 2), b("x_code"), np.uint8), xs=np.full((1, H // 16), b("x_scale"), np.uint8),
               Sx=np.float32(g["Sx"]),
               w13q=np.concatenate([np.full((1, I, H // 2), b("gate_code"), np.uint8),
                                    np.full((1, I, H // 2), b("up_code"), np.uint8)], axis=1),
               w13s=np.concatenate([np.full((1, I, H // 16), b("gate_scale"), np.uint8),
                                    np.full((1, I, H // 16), b("up_scale"), np.uint8)], axis=1),
               Sw13=np.array([g["Sw13"]], np.float32),
               w2q=np.full((1, H, I // 2), b("w2_code"), np.uint8), w2s=np.full((1, H, I // 16), b("w2_scale"), np.uint8),
               Sw2=np.array([g["Sw2"]], np.float32), Sh=np.float32(g["Sh"]),
               ids=np.zeros((1, 1), np.int32), tw=np.ones((1, 1), np.float32))
    out, d = run_moe4(inp, 1, H, I, 1, 1)
    assert np.all(d[0, :I // 2] == b("h_codes")) and np.all(d[0, I // 2:] == b("h_scale"))
    assert np.all(out == b("out_bf16"))


# 128-row tiles with ragged ends, K not a multiple of the 64-element stage,
# several tiles per expert, the one-launch routing (T * topk <= 1024) and the
# four-kernel routing
@pytest.mark.parametrize("T,H,I,E,topk", [(64, 256, 128, 8, 4), (300, 160, 192, 6, 3),
                                          (1, 512, 256, 8, 4), (33, 96, 64, 16, 2),
                                          (700, 128, 128, 4, 2)])
def test_moe4_stagewise(T, H, I, E, topk):
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=T + E)
    out, d = run_moe4(inp, T, H, I, E, topk)
    tokens = np.arange(T) if T <= 64 else np.unique(np.r_[0, 1, np.arange(0, T, 37), T - 1])
    nd = _check_requant(inp, d, T, H, I, topk, tokens)
    assert nd <= max(4, len(tokens) * topk * I // 100), nd
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


# more than 1024 routed rows (four-kernel routing, many tiles per expert),
# a partial last K stage (H = 352: 22 groups) and a partial last column
# block of the down GEMM (H = 352)
@pytest.mark.parametrize("T,H,I,E,topk", [(1100, 352, 384, 6, 2), (600, 256, 128, 3, 2)])
def test_moe4_stagewise_many_tiles(T, H, I, E, topk):
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=T + E)
    out, d = run_moe4(inp, T, H, I, E, topk)
    tokens = np.unique(np.r_[0, 1, np.arange(0, T, 29), T - 1])
    nd = _check_requant(inp, d, T, H, I, topk, tokens)
    assert nd <= max(4, len(tokens) * topk * I // 100), nd
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


def test_moe4_skewed_routing_many_rows():
    """One expert takes most of 1400 routed rows (many tiles, the last one
    ragged), others few or none."""
    T, H, I, E, topk = 700, 128, 256, 8, 2
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=6)
    rng = np.random.default_rng(6)
    ids = np.where(rng.random((T, topk)) < 0.8, 3, rng.integers(0, 4, (T, topk))).astype(np.int32)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 4, ids[:, 1])
    inp["ids"] = ids
    out, d = run_moe4(inp, T, H, I, E, topk)
    tokens = np.arange(0, T, 5)
    _check_requant(inp, d, T, H, I, topk, tokens)
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


def test_moe4_routing_paths_agree():
    """The four-kernel routing and the one-launch routing give the same
    bits: the same tokens routed as 1040 rows (four kernels) and, in a call
    of their own, as the first 1024 of them (one launch) -- the tokens of
    both calls share every expert's weights, and a row's results do not
    depend on the other rows."""
    T, H, I, E, topk = 260, 256, 256, 8, 4
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=21)
    out_big, d_big = run_moe4(inp, T, H, I, E, topk)
    small = dict(inp)
    small["xq"], small["xs"] = inp["xq"][:256], inp["xs"][:256]
    small["ids"], small["tw"] = inp["ids"][:256], inp["tw"][:256]
    out_small, d_small = run_moe4(small, 256, H, I, E, topk)
    assert np.array_equal(d_big[:256 * topk], d_small), "requantised h differs between routing paths"
    assert np.array_equal(out_big[:256], out_small), "output differs between routing paths"


def test_moe4_skewed_routing_and_empty_experts():
    """Half the experts get no tokens, one gets most (several 128-row tiles)."""
    T, H, I, E, topk = 200, 128, 128, 8, 2
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=5)
    rng = np.random.default_rng(5)
    ids = np.where(rng.random((T, topk)) < 0.8, 3, rng.integers(0, 4, (T, topk))).astype(np.int32)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 4, ids[:, 1])
    inp["ids"] = ids
    out, d = run_moe4(inp, T, H, I, E, topk)
    tokens = np.arange(0, T, 3)
    _check_requant(inp, d, T, H, I, topk, tokens)
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


def test_moe4_repeat_bit_identical():
    T, H, I, E, topk = 64, 256, 128, 8, 4
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=9)
    o1, d1 = run_moe4(inp, T, H, I, E, topk)
    o2, d2 = run_moe4(inp, T, H, I, E, topk)
    assert np.array_equal(d1, d2) and np.array_equal(o1, o2)


def test_moe4_full_size_sampled_tokens():
    T, H, I, E, topk = 4096, 4096, 1536, 64, 8
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=0)
    out, d = run_moe4(inp, T, H, I, E, topk)
    tokens = np.array([0, 1, 2048, 4095])
    nd = _check_requant(inp, d, T, H, I, topk, tokens)
    assert nd <= max(4, len(tokens) * topk * I // 100), nd
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)


@pytest.mark.parametrize("T", [5, 300])   # one-launch routing (T * topk <= 1024), four-kernel routing
def test_moe4_out_of_range_ids_dropped(T):
    """Expert ids outside [0, E) (-1 and E here) are dropped: the output is
    the combine of the remaining slots, and a dropped slot's debug row is
    never written."""
    H, I, E, topk = 128, 128, 8, 4
    inp = synth.moe_nvfp4(T, H, I, E, topk, seed=17 + T)
    ids = inp["ids"].copy()
    ids[::2, 1] = -1
    ids[1::3, 3] = E
    inp["ids"] = ids
    out, d = run_moe4(inp, T, H, I, E, topk)
    bad = (ids < 0) | (ids >= E)
    assert bad.any() and np.all(d[bad.ravel()] == 0)
    tokens = np.arange(T) if T <= 64 else np.arange(0, T, 7)
    _check_requant(inp, d, T, H, I, topk, tokens)
    _check_down_combine(inp, d, out, T, H, I, topk, tokens)
