"""Pins of the NVFP4 MoE oracle functions (CPU).

The NVFP4 MoE is the GLU MoE of the FlashInfer swapab_cutedsl_megakernel
skill page (Layout section) with NVFP4 operands.  Each oracle stage is pinned
against something other than itself: the E2M1 encoder against every code and
the tie table of the NVFP4 quantiser reading; the quantiser by round trips of
values already on its grid; gate/up and down against the MXFP8 MoE stages
(pinned by their own hand case) on inputs whose NVFP4 and MXFP8 encodings
decode to the same values; the whole chain by a hand-computed case; and
power-of-two and sign invariants.
"""
import json
import os

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_encoder_codes_and_ties():
    for c, v in enumerate(E2M1):
        assert oracle.enc_e2m1(v) == c
        assert oracle.enc_e2m1(-v) == 8 | c          # -0 keeps its sign bit
    # ties go to the code with a zero low bit (nearest even)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for lo, (v, c) in enumerate(ties.items()):      # v lies midway between codes lo, lo + 1
        assert v == (E2M1[lo] + E2M1[lo + 1]) / 2
        assert oracle.enc_e2m1(v) == c, v
        assert oracle.enc_e2m1(np.nextafter(np.float32(v), np.float32(10))) == lo + 1
        assert oracle.enc_e2m1(np.nextafter(np.float32(v), np.float32(0))) == lo
    for v in (6.5, 7.0, 1e30, float("inf")):
        assert oracle.enc_e2m1(v) == 7 and oracle.enc_e2m1(-v) == 15
    assert oracle.enc_e2m1(float("nan")) == 0


def _dec_nv(codes, scales, S):
    lo, hi = codes & 15, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(-1)
    mag = np.array(E2M1)[c & 7] * np.where(c & 8, -1.0, 1.0)
    return mag * np.repeat([oracle.dec_e4m3(int(b)) for b in scales], 16) * S


def test_nvq_round_trip_on_grid():
    rng = np.random.default_rng(3)
    for S in (1.0, 2.0 ** -8, 0.75):
        for _ in range(50):
            # a group scale byte whose value times 6 * S is representable, and
            # codes whose largest magnitude is 6 (so amax / 6 / S is that value)
            sb = int(rng.integers(0x20, 0x70))
            c = rng.integers(0, 16, 16)
            c[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
            v = (np.array(E2M1)[c & 7] * np.where(c & 8, -1.0, 1.0) * oracle.dec_e4m3(sb) * S)
            v32 = v.astype(np.float32)
            if not np.array_equal(v32.astype(np.float64), v):
                continue
            codes, scales = oracle.nvq(v32, S)
            assert scales[0] == sb
            assert np.array_equal(_dec_nv(codes, scales, S), v)


def test_nvq_zero_and_tiny_groups():
    codes, scales = oracle.nvq(np.zeros(32, np.float32), 1.0)
    assert not codes.any() and not scales.any()
    # amax / 6 below half the smallest E4M3 subnormal (2^-10): scale 0, codes 0
    v = np.full(16, 6 * 2.0 ** -11, np.float32)
    codes, scales = oracle.nvq(v, 1.0)
    assert scales[0] == 0 and not codes.any()


def _mx_from_nv(q, s):
    """NVFP4 codes with group scales 1.0 -> the same values as MXFP8 (E4M3
    codes, E8M0 scale 127), through the E4M3 encoder pinned elsewhere."""
    lo, hi = q & 15, q >> 4
    c = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], -1)
    v = np.array(E2M1)[c & 7] * np.where(c & 8, -1.0, 1.0)
    enc = np.vectorize(lambda x: oracle.enc_e4m3(float(x)))(v).astype(np.uint8)
    return enc, np.full((*q.shape[:-1], q.shape[-1] * 2 // 32), 127, np.uint8)


def test_gateup_and_down_reduce_to_the_mxfp8_stages():
    rng = np.random.default_rng(4)
    T, H, I, E = 2, 64, 64, 2
    one = 0x38
    inp = dict(xq=rng.integers(0, 256, (T, H // 2)).astype(np.uint8), xs=np.full((T, H // 16), one, np.uint8),
               Sx=np.float32(1), w13q=rng.integers(0, 256, (E, 2 * I, H // 2)).astype(np.uint8),
               w13s=np.full((E, 2 * I, H // 16), one, np.uint8), Sw13=np.ones(E, np.float32),
               w2q=rng.integers(0, 256, (E, H, I // 2)).astype(np.uint8),
               w2s=np.full((E, H, I // 16), one, np.uint8), Sw2=np.ones(E, np.float32))
    xq8, xs8 = _mx_from_nv(inp["xq"], inp["xs"])
    w13q8, w13s8 = _mx_from_nv(inp["w13q"], inp["w13s"])
    w2q8, w2s8 = _mx_from_nv(inp["w2q"], inp["w2s"])
    for t in range(T):
        for e in range(E):
            g4, u4, bg4, bu4 = oracle.moe4_gateup(inp, t, e, H, I)
            g8, u8, bg8, bu8 = oracle.moe_gateup(xq8, xs8, t, e, w13q8, w13s8, H, I)
            assert np.array_equal(g4, g8) and np.array_equal(u4, u8)
            assert np.array_equal(bg4, bg8) and np.array_equal(bu4, bu8)
    hq = rng.integers(0, 256, I // 2).astype(np.uint8)
    hs = np.full(I // 16, one, np.uint8)
    hq8, hs8 = _mx_from_nv(hq[None], hs[None])
    for e in range(E):
        y4, by4 = oracle.moe4_down(hq, hs, 1.0, e, inp, H, I)
        y8, by8 = oracle.moe_down(hq8[0], hs8[0], e, w2q8, w2s8, H, I)
        assert np.array_equal(y4, y8) and np.array_equal(by4, by8)


def test_down_scale_and_sign_invariants():
    rng = np.random.default_rng(5)
    H, I, E = 32, 64, 1
    inp = dict(w2q=rng.integers(0, 256, (E, H, I // 2)).astype(np.uint8),
               w2s=rng.integers(0x28, 0x48, (E, H, I // 16)).astype(np.uint8),
               Sw2=np.array([0.375], np.float32))
    hq = rng.integers(0, 256, I // 2).astype(np.uint8)
    hs = rng.integers(0x28, 0x48, I // 16).astype(np.uint8)
    y, _ = oracle.moe4_down(hq, hs, 0.5, 0, inp, H, I)
    y2, _ = oracle.moe4_down(hq, hs, 1.0, 0, inp, H, I)           # Sh doubled
    assert np.array_equal(y2, 2 * y)
    neg = dict(inp, w2q=inp["w2q"] ^ np.uint8(0x88))               # every w2 sign flipped
    yn, _ = oracle.moe4_down(hq, hs, 0.5, 0, neg, H, I)
    assert np.array_equal(yn, -y)


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
    gg, uu, _, _ = oracle.moe4_gateup(inp, 0, 0, H, I)
    hq, hs = oracle.moe4_glu_requant(gg, uu, g["Sh"])
    assert np.all(hq == b("h_codes")) and np.all(hs == b("h_scale"))
    out, _ = oracle.moe4_tokens(inp, 1, H, I, 1, 1, [0])
    assert np.all(out == g["out"])
    assert np.all(oracle.bf16_rne(out) == b("out_bf16"))
