"""Pins of the FP64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against one of: values the pages fix (the
E2M1 -> E4M3 identity of the metrale_circuit hardware::exec module
description), hand-computed worked cases (tests/golden), library routines
(torch's float8 / bfloat16 decoders, numpy integer and float64 matmul, scipy's
logistic function), brute force over every code and scale, and invariants
(sign flip, power-of-two scale).  A dropped term, wrong sign, swapped nibble
or transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import BF16, FP8TOK, MXFP8, NVFP4, Operand

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hexrows(rows):
    return np.array([[int(x, 16) for x in r] for r in rows], dtype=np.uint8)


def _torch_e4m3(b):
    return torch.tensor(np.asarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_e8m0(b):
    return torch.tensor(np.asarray(b, dtype=np.uint8)).view(torch.float8_e8m0fnu).double().numpy()


# -------------------------------------------------------------- decoders
def test_e2m1_identity_golden():
    g = json.load(open(os.path.join(GOLD, "e2m1_to_e4m3_identity.json")))
    for row in g["rows"]:
        c = row["code"]
        conv = oracle.fp8route_convert_word(c << 4) & 0xFF
        assert conv == row["e4m3_byte"], c
        assert oracle.dec_e2m1(c) == row["e2m1_value"], c
        # the pages' claim: E4M3 value of the converted byte is the E2M1 value times 2^-6,
        # decoded here by torch's independent float8_e4m3fn
        assert _torch_e4m3([conv])[0] * 64 == row["e2m1_value"], c
        assert oracle.dec_e4m3(conv) * 64 == oracle.dec_e2m1(c), c
    for w in g["words"]:
        assert oracle.fp8route_convert_word(int(w["in"], 16)) == int(w["out"], 16)


def test_e4m3_decoder_matches_torch_all_codes():
    ref = _torch_e4m3(np.arange(256))
    got = np.array([oracle.dec_e4m3(b) for b in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_e8m0_decoder_matches_torch_all_codes():
    ref = _torch_e8m0(np.arange(256))
    got = np.array([oracle.dec_e8m0(x) for x in range(256)])
    ok = ~np.isnan(ref)
    assert np.isnan(got[255]) and ok.sum() == 255
    assert np.array_equal(ref[ok], got[ok])


def test_bf16_decoder_matches_torch_all_codes():
    u = np.arange(65536, dtype=np.uint16)
    ref = torch.tensor(u.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.dec_bf16(x) for x in range(0, 65536, 7)])
    r = ref[::7]
    assert np.array_equal(np.isnan(r), np.isnan(got))
    assert np.array_equal(r[~np.isnan(r)], got[~np.isnan(got)])


# -------------------------------------------------------------- encoders
def test_e4m3_encoder_matches_torch_in_range_and_ties():
    vals = _torch_e4m3(np.arange(0x7F))          # all finite non-negative grid points
    mids = (vals[:-1] + vals[1:]) / 2             # exact ties
    rng = np.random.default_rng(1)
    rand = rng.uniform(-448, 448, 4000)
    tiny = rng.uniform(-2 ** -6, 2 ** -6, 1000)
    xs = np.concatenate([vals, -vals, mids, -mids, rand, tiny])
    ref = torch.tensor(xs).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.enc_e4m3(x) for x in xs], dtype=np.uint8)
    # +-0: torch keeps the sign of a negative value that rounds to zero, as does the oracle
    assert np.array_equal(got, ref)
    # saturation instead of NaN above the largest finite value
    assert oracle.enc_e4m3(449.0) == 0x7E and oracle.enc_e4m3(-1e9) == 0xFE


def test_bf16_rne_direct_from_fp64():
    # float32-exact inputs: agrees with torch's float -> bfloat16 rounding
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000))).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = oracle.bf16_rne(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # no double rounding: just above a BF16 midpoint by less than a float32 ulp
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert int(oracle.bf16_rne([v])[0]) == 0x3F81
    assert int(oracle.bf16_rne([1.0 + 2.0 ** -8])[0]) == 0x3F80  # exact tie -> even


# ------------------------------------------------------------ hand cases
def _case_operands(c):
    f = c["fmt"]
    if f == "w4a4":
        A = Operand(NVFP4, _hexrows(c["aq"]), _hexrows(c["as"]), tscale=c["Sa"])
        W = Operand(NVFP4, _hexrows(c["wq"]), _hexrows(c["ws"]), tscale=c["Sw"])
    elif f == "w4a8":
        A = Operand(FP8TOK, _hexrows(c["a8"]), rowscale=np.array(c["atok"], np.float32))
        W = Operand(NVFP4, _hexrows(c["wq"]), _hexrows(c["ws"]), tscale=c["Sw"])
    elif f == "w4a16":
        a = np.array([[int(x, 16) for x in r] for r in c["a16"]], dtype=np.uint16)
        A = Operand(BF16, a)
        W = Operand(NVFP4, _hexrows(c["wq"]), _hexrows(c["ws"]), tscale=c["Sw"])
    else:
        A = Operand(MXFP8, _hexrows(c["x"]), _hexrows(c["xs"]))
        W = Operand(MXFP8, _hexrows(c["w"]), _hexrows(c["wsx"]))
    return A, W


HAND = json.load(open(os.path.join(GOLD, "hand_cases.json")))["cases"]


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_cases(case):
    A, W = _case_operands(case)
    Cv, Bv = oracle.gemm_full(A, W, nthreads=1)
    assert np.array_equal(Cv, np.array(case["C"]))
    bits = oracle.bf16_rne(Cv)
    assert np.array_equal(bits, np.array([[int(x, 16) for x in r] for r in case["bf16"]]))
    assert np.all(Bv >= np.abs(Cv))


# --------------------------------------- exact-FP8 route == declared W4A4
def test_fp8route_w4a4_exhaustive_single_group():
    """Every E2M1 code pair x every finite non-negative E4M3 scale pair, one
    16-element group: the emulated FP8 route returns exactly the declared
    product (each group term is exact in FP32)."""
    codes = np.arange(16, dtype=np.uint8)
    scales = np.arange(0x7F, dtype=np.uint8)          # 0x00..0x7E
    ca, cw, sa, sw = np.meshgrid(codes, codes, scales, scales, indexing="ij")
    ca, cw, sa, sw = (x.ravel() for x in (ca, cw, sa, sw))
    n = ca.size
    # vary the 16 elements: element k uses code (c + k) mod 16 so both signs appear
    k = np.arange(16, dtype=np.uint8)
    ea = (ca[:, None] + k[None, :]) % 16
    ew = (cw[:, None] + 3 * k[None, :]) % 16
    aq = (ea[:, 0::2] | (ea[:, 1::2] << 4)).astype(np.uint8)
    wq = (ew[:, 0::2] | (ew[:, 1::2] << 4)).astype(np.uint8)
    emu = oracle.fp8route_w4a4_rows(aq, sa[:, None], wq, sw[:, None])
    A = Operand(NVFP4, aq, sa[:, None].copy())
    W = Operand(NVFP4, wq, sw[:, None].copy())
    idx = np.arange(n)
    Cd, _ = oracle.gemm_points(A, W, idx, idx)
    assert np.array_equal(emu.astype(np.float64), Cd), np.where(emu != Cd)[0][:5]


def test_fp8route_w4a4_random_multigroup():
    rng = np.random.default_rng(3)
    for K in (64, 256):
        aq = rng.integers(0, 256, (2, K // 2), dtype=np.uint8)
        wq = rng.integers(0, 256, (2, K // 2), dtype=np.uint8)
        as_ = rng.integers(0, 0x7F, (2, K // 16), dtype=np.uint8)
        ws = rng.integers(0, 0x7F, (2, K // 16), dtype=np.uint8)
        A, W = Operand(NVFP4, aq, as_), Operand(NVFP4, wq, ws)
        Cd, Bd = oracle.gemm_full(A, W)
        for m in range(2):
            for n_ in range(2):
                emu = oracle.fp8route_w4a4_point(aq[m], as_[m], wq[n_], ws[n_])
                # only the cross-group FP32 additions round
                assert abs(emu - Cd[m, n_]) <= 2.0 ** -24 * (K // 16) * Bd[m, n_]


def test_fp8route_w4a8_exhaustive_single_group():
    a8 = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
    codes = np.arange(16, dtype=np.uint8)
    scales = np.arange(0x7F, dtype=np.uint8)
    A8, CW, SW = (x.ravel() for x in np.meshgrid(a8, codes, scales, indexing="ij"))
    k = np.arange(16, dtype=np.uint8)
    ew = (CW[:, None] + 5 * k[None, :]) % 16
    wq = (ew[:, 0::2] | (ew[:, 1::2] << 4)).astype(np.uint8)
    arow = np.repeat(A8[:, None], 16, axis=1)
    emu = oracle.fp8route_w4a8_rows(arow, wq, SW[:, None])
    A = Operand(FP8TOK, arow, rowscale=np.ones(A8.size, np.float32))
    W = Operand(NVFP4, wq, SW[:, None].copy())
    idx = np.arange(A8.size)
    Cd, _ = oracle.gemm_points(A, W, idx, idx)
    assert np.array_equal(emu.astype(np.float64), Cd)


# -------------------------------------------- library / closed-form checks
E2M1_TABLE = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])  # OCP MX


def _indep_nvfp4(q, s):
    """NVFP4 decode built from the OCP E2M1 table and torch's E4M3 decoder."""
    c = np.empty((q.shape[0], q.shape[1] * 2), np.int64)
    c[:, 0::2] = q & 15
    c[:, 1::2] = q >> 4
    return E2M1_TABLE[c] * np.repeat(_torch_e4m3(s), 16, axis=1)


def test_nvfp4_pairs_match_float64_matmul():
    rng = np.random.default_rng(4)
    M, N, K = 7, 9, 96
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    Sa, Sw = 0.37, 1.9
    a, w = _indep_nvfp4(aq, as_), _indep_nvfp4(wq, ws)
    ref = Sa * Sw * (torch.tensor(a) @ torch.tensor(w).T).numpy()
    Cv, Bv = oracle.gemm_full(Operand(NVFP4, aq, as_, tscale=Sa), Operand(NVFP4, wq, ws, tscale=Sw))
    assert np.allclose(Cv, ref, rtol=0, atol=1e-12 * Bv.max())
    ref_b = Sa * Sw * (np.abs(a) @ np.abs(w).T)
    assert np.allclose(Bv, ref_b, rtol=1e-12)
    # W4A8: FP8 activations with per-token scales
    a8 = rng.integers(0, 0x7F, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    atok = rng.uniform(0.1, 2, M).astype(np.float32)
    ref = (atok[:, None].astype(np.float64) * Sw) * (_torch_e4m3(a8) @ w.T)
    Cv, Bv = oracle.gemm_full(Operand(FP8TOK, a8, rowscale=atok), Operand(NVFP4, wq, ws, tscale=Sw))
    assert np.allclose(Cv, ref, rtol=0, atol=1e-12 * Bv.max())
    # W4A16: BF16 activations
    a16 = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    af = torch.tensor(a16.view(np.int16)).view(torch.bfloat16).double().numpy()
    Cv, Bv = oracle.gemm_full(Operand(BF16, a16), Operand(NVFP4, wq, ws, tscale=Sw))
    assert np.allclose(Cv, Sw * (af @ w.T), rtol=0, atol=1e-12 * Bv.max())


def test_bf16_and_mxfp8_match_float64_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 5, 6, 64
    a16 = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w16 = synth.to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    af = torch.tensor(a16.view(np.int16)).view(torch.bfloat16).double()
    wf = torch.tensor(w16.view(np.int16)).view(torch.bfloat16).double()
    Cv, Bv = oracle.gemm_full(Operand(BF16, a16), Operand(BF16, w16))
    assert np.allclose(Cv, (af @ wf.T).numpy(), rtol=0, atol=1e-13 * Bv.max())
    xq = rng.integers(0, 0x7F, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    wq = rng.integers(0, 0x7F, (N, K), dtype=np.uint8)
    xs = rng.integers(110, 140, (M, K // 32), dtype=np.uint8)
    wsx = rng.integers(110, 140, (N, K // 32), dtype=np.uint8)
    xv = _torch_e4m3(xq) * np.repeat(_torch_e8m0(xs), 32, axis=1)
    wv = _torch_e4m3(wq) * np.repeat(_torch_e8m0(wsx), 32, axis=1)
    Cv, Bv = oracle.gemm_full(Operand(MXFP8, xq, xs), Operand(MXFP8, wq, wsx))
    assert np.allclose(Cv, xv @ wv.T, rtol=0, atol=1e-13 * Bv.max())


def test_exact_sum_regime_integer_matmul():
    """Small integers: every partial sum is exact, so the oracle equals an
    integer matmul exactly.  NVFP4 with scale 1 and S = 1: twice each value
    is an integer given by the OCP table, with element 2i in the low nibble."""
    rng = np.random.default_rng(6)
    M, N, K = 8, 8, 64
    ai = rng.integers(-8, 9, (M, K))
    wi = rng.integers(-8, 9, (N, K))
    a16 = synth.to_bf16_bits(ai.astype(np.float32))
    w16 = synth.to_bf16_bits(wi.astype(np.float32))
    Cv, _ = oracle.gemm_full(Operand(BF16, a16), Operand(BF16, w16))
    assert np.array_equal(Cv, (ai @ wi.T).astype(np.float64))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12])
    ca = rng.integers(0, 16, (M, K))
    cw = rng.integers(0, 16, (N, K))
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)  # noqa: E731
    ones = lambda r: np.full((r, K // 16), 0x38, np.uint8)  # noqa: E731
    Cv, _ = oracle.gemm_full(Operand(NVFP4, pack(ca), ones(M)), Operand(NVFP4, pack(cw), ones(N)))
    assert np.array_equal(Cv * 4, (twice[ca] @ twice[cw].T).astype(np.float64))


def test_invariants_sign_and_power_of_two():
    rng = np.random.default_rng(7)
    M, N, K = 4, 5, 64
    aq = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    as_ = rng.integers(0x08, 0x70, (M, K // 16), dtype=np.uint8)
    wq = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x08, 0x70, (N, K // 16), dtype=np.uint8)
    A = Operand(NVFP4, aq, as_, tscale=0.7)
    C0, _ = oracle.gemm_full(A, Operand(NVFP4, wq, ws, tscale=1.3))
    wq2 = wq.copy()
    wq2[2] ^= 0x88                      # flip the sign bit of both nibbles of row 2
    C1, _ = oracle.gemm_full(A, Operand(NVFP4, wq2, ws, tscale=1.3))
    assert np.array_equal(C1[:, 2], -C0[:, 2])
    assert np.array_equal(np.delete(C1, 2, 1), np.delete(C0, 2, 1))
    ws2 = ws.copy()
    ws2[3] += 8                          # E4M3 exponent field + 1 (no overflow below 0x70)
    C2, _ = oracle.gemm_full(A, Operand(NVFP4, wq, ws2, tscale=1.3))
    assert np.array_equal(C2[:, 3], 2 * C0[:, 3])
    # transposition: swapping the operands transposes C (same format both sides)
    Ct, _ = oracle.gemm_full(Operand(NVFP4, wq, ws, tscale=1.3), A)
    assert np.array_equal(Ct, C0.T)


# ------------------------------------------------------------------- MXFP8
def test_mxq_matches_independent_quantiser():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(32 * 200) * np.exp(rng.uniform(-20, 20, 32 * 200))).astype(np.float32)
    v[:32] = 0.0                                     # an all-zero block
    v[32:64] = 2.0 ** -140                           # clamped exponent
    c1, s1 = oracle.mxq(v)
    c2, s2 = synth.quant_mxfp8(v.reshape(1, -1))
    assert np.array_equal(s1, s2.ravel()) and np.array_equal(c1, c2.ravel())
    # round trip, per regime of the scaled value s = v / 2^X
    scale = np.repeat(_torch_e8m0(s1), 32)
    dec = _torch_e4m3(c1) * scale
    sv = v.astype(np.float64) / scale
    normal = (np.abs(sv) >= 2.0 ** -6) & (np.abs(sv) <= 448)
    assert np.all(np.abs(dec - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    sub = np.abs(sv) < 2.0 ** -6
    assert np.all(np.abs(dec - v)[sub] <= 2.0 ** -10 * scale[sub])
    sat = np.abs(sv) > 448
    assert np.all(np.abs(dec[sat]) == 448 * scale[sat])
    assert normal.sum() > 1000


def test_mxq_hand_cases():
    """The MX exponent rule and element rounding against hand derivations from
    the OCP MX conversion rule (tests/golden/mx_quant_hand.json), including a
    block whose code changes if the exponent offset is 7 instead of 8, ties
    to the even mantissa, saturation, the all-zero block and small values."""
    g = json.load(open(os.path.join(GOLD, "mx_quant_hand.json")))
    for blk in g["blocks"]:
        v = np.zeros(32, np.float32)
        for k, x in blk["values"].items():
            v[int(k)] = x
        codes, scales = oracle.mxq(v)
        want = np.zeros(32, np.uint8)
        for k, c in blk["codes"].items():
            want[int(k)] = int(c, 16)
        assert scales[0] == blk["scale"], blk["derivation"]
        assert np.array_equal(codes, want), (codes, blk["derivation"])


def _moe_hand_inputs(g):
    H, I = g["H"], g["I"]
    return dict(
        xq=np.full((1, H), int(g["x_code"], 16), np.uint8),
        xs=np.full((1, H // 32), g["x_scale"], np.uint8),
        w13q=np.concatenate([np.full((1, I, H), int(g["gate_code"], 16), np.uint8),
                             np.full((1, I, H), int(g["up_code"], 16), np.uint8)], axis=1),
        w13s=np.full((1, 2 * I, H // 32), g["w13_scale"], np.uint8),
        w2q=np.full((1, H, I), int(g["w2_code"], 16), np.uint8),
        w2s=np.full((1, H, I // 32), g["w2_scale"], np.uint8),
        ids=np.zeros((1, 1), np.int32), tw=np.ones((1, 1), np.float32))


@pytest.mark.parametrize("name", ["moe_hand.json", "moe_hand_128.json"])
def test_moe_hand_cases(name):
    """Hand-computed one-token MXFP8 MoE cases: every stage of the oracle
    (gate/up, GLU, MX re-quantisation, down, combine, BF16) against the
    derivation in the golden file."""
    g = json.load(open(os.path.join(GOLD, name)))
    H, I = g["H"], g["I"]
    inp = _moe_hand_inputs(g)
    gg, u, _, _ = oracle.moe_gateup(inp["xq"], inp["xs"], 0, 0, inp["w13q"], inp["w13s"], H, I)
    hq, hs = oracle.moe_glu_requant(gg, u)
    assert np.all(hq == int(g["h_code"], 16)) and np.all(hs == g["h_scale"]), (hq[:4], hs)
    y, _ = oracle.moe_down(hq, hs, 0, inp["w2q"], inp["w2s"], H, I)
    assert np.all(y == g["out"])
    o64, _ = oracle.moe_tokens(inp, 1, H, I, 1, 1, [0])
    assert np.all(o64 == g["out"])
    assert oracle.bf16_rne(np.array([g["out"]]))[0] == int(g["out_bf16"], 16)


# --------------------------------------------------------------------- MoE
def _tiny_moe(seed=9, T=6, H=64, I=64, E=3, topk=2):
    inp = synth.moe(T, H, I, E, topk, seed=seed, w_std=0.2)
    return inp, (T, H, I, E, topk)


def test_moe_gateup_and_down_one_hot():
    inp, (T, H, I, E, topk) = _tiny_moe()
    xq = np.zeros((1, H), np.uint8)
    xq[0, 5] = 0x38                                   # x = e_5 (scale 1.0)
    xs = np.full((1, H // 32), 127, np.uint8)
    g, u, _, _ = oracle.moe_gateup(xq, xs, 0, 1, inp["w13q"], inp["w13s"], H, I)
    w13 = _torch_e4m3(inp["w13q"][1]) * np.repeat(_torch_e8m0(inp["w13s"][1]), 32, axis=1)
    assert np.array_equal(g, w13[:I, 5]) and np.array_equal(u, w13[I:, 5])
    hq = np.zeros(I, np.uint8)
    hq[7] = 0x40                                      # h = 2 * e_7
    hs = np.full(I // 32, 127, np.uint8)
    y, _ = oracle.moe_down(hq, hs, 2, inp["w2q"], inp["w2s"], H, I)
    w2 = _torch_e4m3(inp["w2q"][2]) * np.repeat(_torch_e8m0(inp["w2s"][2]), 32, axis=1)
    assert np.array_equal(y, 2 * w2[:, 7])


def test_moe_glu_requant_matches_library_silu():
    from scipy.special import expit
    rng = np.random.default_rng(10)
    I = 256
    g = rng.standard_normal(I) * 3
    u = rng.standard_normal(I) * 2
    hq, hs = oracle.moe_glu_requant(g, u)
    h = (g * expit(g) * u).astype(np.float32)
    c2, s2 = synth.quant_mxfp8(h.reshape(1, -1))
    assert np.array_equal(hs, s2.ravel())
    assert np.array_equal(hq, c2.ravel())
    assert oracle.moe_glu_requant(np.zeros(32), np.ones(32))[0].max() == 0  # silu(0) = 0


def test_moe_tokens_composition_and_linearity():
    inp, (T, H, I, E, topk) = _tiny_moe()
    out, bound = oracle.moe_tokens(inp, T, H, I, E, topk, np.arange(T))
    # composition of the stage functions, slots in ascending order
    t = 3
    ref = np.zeros(H)
    for j in range(topk):
        e = int(inp["ids"][t, j])
        g, u, _, _ = oracle.moe_gateup(inp["xq"], inp["xs"], t, e, inp["w13q"], inp["w13s"], H, I)
        hq, hs = oracle.moe_glu_requant(g, u)
        y, _ = oracle.moe_down(hq, hs, e, inp["w2q"], inp["w2s"], H, I)
        ref += float(inp["tw"][t, j]) * y
    assert np.array_equal(out[t], ref)
    assert np.all(bound >= np.abs(out))
    # the same expert in both slots with weights 1/4 and 3/4 equals one slot of weight 1
    inp2 = dict(inp)
    inp2["ids"] = np.repeat(inp["ids"][:, :1], 2, axis=1).copy()
    inp2["tw"] = np.tile(np.array([0.25, 0.75], np.float32), (T, 1))
    o2, _ = oracle.moe_tokens(inp2, T, H, I, E, 2, np.arange(T))
    inp1 = dict(inp)
    inp1["ids"] = inp["ids"][:, :1].copy()
    inp1["tw"] = np.ones((T, 1), np.float32)
    o1, _ = oracle.moe_tokens(inp1, T, H, I, E, 1, np.arange(T))
    assert np.allclose(o2, o1, rtol=1e-15, atol=1e-300)


def test_oracle_rejects_bad_arguments():
    a = Operand(NVFP4, np.zeros((2, 8), np.uint8), np.zeros((2, 1), np.uint8))
    w = Operand(NVFP4, np.zeros((2, 16), np.uint8), np.zeros((2, 2), np.uint8))
    with pytest.raises(ValueError):
        oracle.gemm_full(a, w)                        # K mismatch
    with pytest.raises(ValueError):
        oracle.gemm_points(a, a, [0], [5])            # out of range point
