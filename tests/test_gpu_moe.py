"""GPU parity of the MXFP8 grouped MoE GLU against the FP64 oracle.

The re-quantisation of h inside the path is a decision point: where h lies on
an E4M3 rounding boundary (or its block amax on a power of two), a correct
FP32 kernel and the FP64 oracle can pick neighbouring codes.  Parity is
therefore checked stage-wise:
  (ii)  the kernel's re-quantised h (debug tap) equals the oracle's, except
        codes whose oracle value lies within the FP32 accumulation bound of a
        rounding boundary -- each such case a single-step difference;
  (iii) the kernel's output equals the oracle's down projection and combine
        applied to the kernel's own h: FP32 tolerance / 1 BF16 ulp.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from checks import fp8_window_bound

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_scaled_precision_tn_amd as mg
    mg.load()
    yield


def run_moe(inp, T, H, I, E, topk, dbg=True, gu=False):
    """Output bits [T,H], the re-quantised h rows (dbg) and, with gu, the FP32
    gate/up accumulator rows [T*topk, 2I] as well."""
    import block_scaled_precision_tn_amd as mg
    from gpu_cases import dev
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    dbg_h = torch.zeros(T * topk * (I + I // 32), dtype=torch.uint8, device="cuda") if dbg else None
    dbg_gu = torch.zeros(T * topk * 2 * I, dtype=torch.float32, device="cuda") if gu else None
    mg.mgemm_moe_mxfp8_glu(dev(inp["xq"]), dev(inp["xs"]), dev(inp["ids"]), dev(inp["tw"]),
                           dev(inp["w13q"]), dev(inp["w13s"]), dev(inp["w2q"]), dev(inp["w2s"]),
                           out, dbg_h=dbg_h, dbg_gu=dbg_gu)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    d = dbg_h.cpu().numpy().reshape(T * topk, I + I // 32) if dbg else None
    if gu:
        return o, d, dbg_gu.cpu().numpy().reshape(T * topk, 2 * I)
    return o, d


def _check_gateup(inp, gu, T, H, I, topk, tokens=None):
    """Stage (i): the kernel's FP32 gate/up accumulators against the oracle's
    g and u, within 1e-5 * sum|x w| plus the MX MFMA's summation-window
    allowance.  Returns the largest err / (1e-5 B)."""
    from checks import check_f32
    worst = 0.0
    for t in (range(T) if tokens is None else tokens):
        for j in range(topk):
            e = int(inp["ids"][t, j])
            if not 0 <= e < inp["w13q"].shape[0]:
                continue
            g, u, bg, bu = oracle.moe_gateup(inp["xq"], inp["xs"], t, e, inp["w13q"], inp["w13s"], H, I)
            hw = mx_window(inp["xq"][t][None, :], inp["xs"][t][None, :], inp["w13q"][e], inp["w13s"][e])
            row = gu[t * topk + j]
            worst = max(worst, check_f32(row, np.r_[g, u], np.r_[bg, bu], what=f"gate/up {t},{j}",
                                         extra=hw))
    return worst


def test_moe_hand_case():
    g = json.load(open(os.path.join(GOLD, "moe_hand.json")))
    H, I = g["H"], g["I"]
    inp = dict(
        xq=np.full((1, H), int(g["x_code"], 16), np.uint8),
        xs=np.full((1, H // 32), g["x_scale"], np.uint8),
        w13q=np.concatenate([np.full((1, I, H), int(g["gate_code"], 16), np.uint8),
                             np.full((1, I, H), int(g["up_code"], 16), np.uint8)], axis=1),
        w13s=np.full((1, 2 * I, H // 32), g["w13_scale"], np.uint8),
        w2q=np.full((1, H, I), int(g["w2_code"], 16), np.uint8),
        w2s=np.full((1, H, I // 32), g["w2_scale"], np.uint8),
        ids=np.zeros((1, 1), np.int32), tw=np.ones((1, 1), np.float32))
    out, d = run_moe(inp, 1, H, I, 1, 1)
    assert np.all(d[0, :I] == int(g["h_code"], 16)) and np.all(d[0, I:] == g["h_scale"])
    assert np.all(out == int(g["out_bf16"], 16))
    # the oracle agrees on the same case
    o64, _ = oracle.moe_tokens(inp, 1, H, I, 1, 1, [0])
    assert np.all(o64 == g["out"])


def _e4m3_val(b):
    return torch.tensor(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _e4m3_half_step(v):
    """Half the E4M3 spacing at |v| (v on the E4M3 grid, in scaled units)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 0.5 * 2.0 ** (e - 3)


def _check_requant(inp, d, T, H, I, topk, tol=1e-5, tokens=None):
    """Stage (ii).  Where the GPU's h code/scale equal the oracle's, nothing to
    check.  Elsewhere each GPU code must be a correct MX rounding of some h'
    with |h' - h| <= dh, dh being the bound implied by the FP32 accumulation
    tolerance 1e-5 * sum|x w| on g and u (first order through silu(g) * u).
    Checks every token, or the given ones.  Returns the number of such codes."""
    from scipy.special import expit
    n_diff = 0
    for t in (range(T) if tokens is None else tokens):
        for j in range(topk):
            e = int(inp["ids"][t, j])
            if not 0 <= e < inp["w13q"].shape[0]:
                continue                         # a dropped slot
            g, u, bg, bu = oracle.moe_gateup(inp["xq"], inp["xs"], t, e, inp["w13q"], inp["w13s"], H, I)
            hq, hs = oracle.moe_glu_requant(g, u)
            gq, gs = d[t * topk + j, :I], d[t * topk + j, I:]
            if np.array_equal(hq, gq) and np.array_equal(hs, gs):
                continue
            s = expit(g)
            dsilu = s * (1 + g * (1 - s))
            h = g * s * u
            hw = mx_window(inp["xq"][t][None, :], inp["xs"][t][None, :], inp["w13q"][e],
                           inp["w13s"][e])
            eg = tol * bg + hw[:I]
            eu = tol * bu + hw[I:]
            dh = np.abs(dsilu * u) * eg + np.abs(g * s) * eu + 4 * 2.0 ** -24 * np.abs(h)
            for b in range(I // 32):
                sl = slice(32 * b, 32 * b + 32)
                if hs[b] != gs[b]:
                    # block scales differ only where the block amax straddles a power of two
                    amax = np.max(np.abs(h[sl]))
                    p2 = 2.0 ** np.round(np.log2(amax))
                    assert abs(amax - p2) <= np.max(dh[sl]) * 2, (t, j, b, amax, hs[b], gs[b])
                    assert abs(int(hs[b]) - int(gs[b])) == 1
                X = float(gs[b]) - 127
                vg = _e4m3_val(gq[sl]) * 2.0 ** X                 # GPU h, decoded
                hstep = _e4m3_half_step(_e4m3_val(gq[sl])) * 2.0 ** X
                sat = np.abs(_e4m3_val(gq[sl])) == 448
                ok = (np.abs(vg - h[sl]) <= hstep + dh[sl] * 2) | \
                     (sat & (np.abs(h[sl]) * 2.0 ** -X >= 448 - dh[sl] * 2.0 ** -X * 2))
                assert ok.all(), (t, j, b, np.where(~ok)[0], h[sl][~ok], vg[~ok], dh[sl][~ok])
                n_diff += int((gq[sl] != hq[sl]).sum())
    return n_diff


def mx_window(qa, sa, qw, sw):
    """FP8 MFMA summation-window allowance (fp8_window_bound) of MXFP8 dot
    products: the MX MFMA multiplies the E4M3 codes, and a group of 8's sum is
    then scaled by the two E8M0 block scales of its 32-element block.
    qa/sa: codes [.., K] and scales [.., K/32] of one side, qw/sw the other's
    (broadcastable); returns the allowance per leading index."""
    e8 = lambda s: torch.tensor(np.asarray(s, np.uint8)).view(torch.float8_e8m0fnu).double().numpy()  # noqa: E731
    g = np.repeat(e8(sa) * e8(sw), 4, axis=-1)
    return fp8_window_bound(_e4m3_val(qa), _e4m3_val(qw), g)


def _check_down_combine(inp, d, out, T, H, I, topk, tokens):
    """Stage (iii): oracle down projection + combine applied to the GPU's h.
    Tolerance: 1e-5 * sum|w y-terms| plus the FP8 MFMA window term of every
    slot's down-projection sum, plus the FP32 rounding of the combine."""
    from gpu_cases import check_bf16_vs
    ref = np.zeros((len(tokens), H))
    bnd = np.zeros((len(tokens), H))
    extra = np.zeros((len(tokens), H))
    for ti, t in enumerate(tokens):
        for j in range(topk):
            e = int(inp["ids"][t, j])
            if not 0 <= e < inp["w13q"].shape[0]:
                continue                         # a dropped slot
            row = d[t * topk + j]
            y, by = oracle.moe_down(row[:I].copy(), row[I:].copy(), e, inp["w2q"], inp["w2s"], H, I)
            w = float(inp["tw"][t, j])
            ref[ti] += w * y
            bnd[ti] += abs(w) * by
            extra[ti] += abs(w) * mx_window(row[:I][None, :], row[I:][None, :], inp["w2q"][e],
                                            inp["w2s"][e])
        extra[ti] += topk * 2.0 ** -23 * bnd[ti]
    check_bf16_vs(out[tokens], ref, bnd, what="moe out", extra=extra)


# More than 32 tokens take the grouped kernels: with H and I multiples of 512
# the 256 x 256 tiles (tile list of 256 rows), otherwise 128 x 128 tiles,
# where H or I a multiple of 512 takes the chunked scale loads (16 bytes of a
# scale row per lane for 8 stages) and the others the per-stage 2-byte
# loads.  Up to 32 tokens with H and I multiples of 128 take the
# decode-sized (swap-AB) kernels.
@pytest.mark.parametrize("T,H,I,E,topk", [(64, 256, 128, 8, 4), (300, 128, 192, 6, 3),
                                          (33, 64, 64, 16, 2), (40, 1024, 512, 4, 2),
                                          (300, 512, 512, 4, 2), (160, 512, 1024, 8, 2),
                                          (24, 512, 1536, 3, 2), (1, 512, 256, 8, 4),
                                          (7, 256, 384, 16, 3), (32, 1024, 512, 8, 2),
                                          (16, 128, 128, 64, 8), (5, 64, 128, 4, 2)])
def test_moe_stagewise(T, H, I, E, topk):
    inp = synth.moe(T, H, I, E, topk, seed=T + E)
    out, d, gu = run_moe(inp, T, H, I, E, topk, gu=True)
    worst = _check_gateup(inp, gu, T, H, I, topk)
    print(f"[parity] moe {T}x{H}x{I} E={E} top{topk}: gate/up max err/B {worst:.3g}")
    nb = _check_requant(inp, d, T, H, I, topk)
    assert nb <= max(4, T * topk * I // 100), nb   # differing codes are rare
    _check_down_combine(inp, d, out, T, H, I, topk, np.arange(T))


def test_moe_skewed_routing_and_empty_experts():
    """Half the experts get no tokens, one gets most (several 128-row tiles)."""
    T, H, I, E, topk = 200, 128, 128, 8, 2
    inp = synth.moe(T, H, I, E, topk, seed=5)
    rng = np.random.default_rng(5)
    ids = np.where(rng.random((T, topk)) < 0.8, 3, rng.integers(0, 4, (T, topk))).astype(np.int32)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 4, ids[:, 1])
    inp["ids"] = ids
    out, d = run_moe(inp, T, H, I, E, topk)
    _check_requant(inp, d, T, H, I, topk)
    _check_down_combine(inp, d, out, T, H, I, topk, np.arange(T))


def test_moe_skewed_routing_big_tiles():
    """The 256-row tiles: one expert holds a full tile and a partial one,
    another one partial tile, the rest 1 to 35 rows (tiles whose idle waves
    skip their MFMAs) or none."""
    T, H, I, E, topk = 300, 512, 512, 8, 2
    inp = synth.moe(T, H, I, E, topk, seed=6)
    rng = np.random.default_rng(6)
    ids = np.where(rng.random((T, topk)) < 0.85, 3, rng.integers(0, 3, (T, topk))).astype(np.int32)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 5) % E, ids[:, 1])
    inp["ids"] = ids
    out, d, gu = run_moe(inp, T, H, I, E, topk, gu=True)
    _check_gateup(inp, gu, T, H, I, topk)
    _check_requant(inp, d, T, H, I, topk)
    _check_down_combine(inp, d, out, T, H, I, topk, np.arange(T))


def test_moe_hand_case_decode_kernels():
    """The hand case at H = I = 128 (one token: the decode-sized kernels)."""
    g = json.load(open(os.path.join(GOLD, "moe_hand_128.json")))
    H, I = g["H"], g["I"]
    inp = dict(
        xq=np.full((1, H), int(g["x_code"], 16), np.uint8),
        xs=np.full((1, H // 32), g["x_scale"], np.uint8),
        w13q=np.concatenate([np.full((1, I, H), int(g["gate_code"], 16), np.uint8),
                             np.full((1, I, H), int(g["up_code"], 16), np.uint8)], axis=1),
        w13s=np.full((1, 2 * I, H // 32), g["w13_scale"], np.uint8),
        w2q=np.full((1, H, I), int(g["w2_code"], 16), np.uint8),
        w2s=np.full((1, H, I // 32), g["w2_scale"], np.uint8),
        ids=np.zeros((1, 1), np.int32), tw=np.ones((1, 1), np.float32))
    out, d = run_moe(inp, 1, H, I, 1, 1)
    assert np.all(d[0, :I] == int(g["h_code"], 16)) and np.all(d[0, I:] == g["h_scale"])
    assert np.all(out == int(g["out_bf16"], 16))
    o64, _ = oracle.moe_tokens(inp, 1, H, I, 1, 1, [0])
    assert np.all(o64 == g["out"])


def test_moe_decode_expert_named_twice():
    """Few tokens, each naming expert 0 in two slots: expert 0 gets more than
    32 rows, which the decode-sized kernels take 32 at a time."""
    T, H, I, E, topk = 20, 256, 256, 4, 4
    inp = synth.moe(T, H, I, E, topk, seed=11)
    ids = np.zeros((T, topk), np.int32)
    ids[:, 2] = 1 + np.arange(T) % 3
    ids[:, 3] = np.arange(T) % 4
    inp["ids"] = ids
    out, d = run_moe(inp, T, H, I, E, topk)
    _check_requant(inp, d, T, H, I, topk)
    _check_down_combine(inp, d, out, T, H, I, topk, np.arange(T))


@pytest.mark.parametrize("T", [3, 32])
def test_moe_decode_repeat_bit_identical(T):
    H, I, E, topk = 256, 256, 8, 4
    inp = synth.moe(T, H, I, E, topk, seed=12)
    o1, d1 = run_moe(inp, T, H, I, E, topk)
    o2, d2 = run_moe(inp, T, H, I, E, topk)
    assert np.array_equal(d1, d2)
    assert np.array_equal(o1, o2)


def test_moe_repeat_bit_identical():
    """The combine adds a token's slots in a fixed order (no atomics), and
    the row order inside an expert does not change any row's result: repeats
    are bit-identical."""
    T, H, I, E, topk = 64, 256, 128, 8, 4
    inp = synth.moe(T, H, I, E, topk, seed=9)
    o1, d1 = run_moe(inp, T, H, I, E, topk)
    o2, d2 = run_moe(inp, T, H, I, E, topk)
    assert np.array_equal(d1, d2)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("T", [5, 40])   # one-workgroup routing (decode kernels), four-kernel routing
def test_moe_out_of_range_ids_dropped(T):
    """Expert ids outside [0, E) (-1 and E here) are dropped: the output is
    the combine of the remaining slots, and a dropped slot's debug row is
    never written."""
    H, I, E, topk = 256, 128, 8, 4
    inp = synth.moe(T, H, I, E, topk, seed=13 + T)
    ids = inp["ids"].copy()
    ids[::2, 1] = -1
    ids[1::3, 3] = E
    inp["ids"] = ids
    out, d = run_moe(inp, T, H, I, E, topk)
    bad = (ids < 0) | (ids >= E)
    assert bad.any() and np.all(d[bad.ravel()] == 0)
    _check_requant(inp, d, T, H, I, topk)
    _check_down_combine(inp, d, out, T, H, I, topk, np.arange(T))
