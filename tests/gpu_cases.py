"""Shared helpers for the GPU parity tests: run each entry point of the HIP
library through the Python binding on given bytes, and compute the oracle's
answer for the same bytes.  Test infrastructure only."""
import numpy as np
import torch

import block_scaled_precision_tn_amd as mg
import oracle
from oracle import BF16, FP8TOK, MXFP8, NVFP4, Operand

from checks import check_bf16, check_f32, fp8_window_bound


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def scalar(v):
    return torch.tensor([float(v)], dtype=torch.float32, device="cuda")


def out_tensor(M, N, f32):
    return torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")


def to_np(c):
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).cpu().numpy().view(np.uint16)
    return c.cpu().numpy()


# ------------------------------------------------------------ GPU runners
def gpu_w4a4(inp, f32):
    M, N = inp["aq"].shape[0], inp["wq"].shape[0]
    C = out_tensor(M, N, f32)
    mg.mgemm_w4a4(dev(inp["aq"]), dev(inp["as_"]), scalar(inp["Sa"]), dev(inp["wq"]),
                  dev(inp["ws"]), scalar(inp["Sw"]), C)
    torch.cuda.synchronize()
    return to_np(C)


def gpu_w4a8(inp, f32):
    M, N = inp["aq"].shape[0], inp["wq"].shape[0]
    C = out_tensor(M, N, f32)
    mg.mgemm_w4a8(dev(inp["aq"]), dev(inp["atok"]), dev(inp["wq"]), dev(inp["ws"]),
                  scalar(inp["Sw"]), C)
    torch.cuda.synchronize()
    return to_np(C)


def gpu_w4a16(inp, f32):
    M, N = inp["a"].shape[0], inp["wq"].shape[0]
    C = out_tensor(M, N, f32)
    mg.mgemm_w4a16(dev(inp["a"].view(np.int16), torch.bfloat16), dev(inp["wq"]), dev(inp["ws"]),
                   scalar(inp["Sw"]), C)
    torch.cuda.synchronize()
    return to_np(C)


def gpu_bf16(inp, f32):
    M, N = inp["a"].shape[0], inp["w"].shape[0]
    C = out_tensor(M, N, f32)
    mg.mgemm_bf16(dev(inp["a"].view(np.int16), torch.bfloat16),
                  dev(inp["w"].view(np.int16), torch.bfloat16), C)
    torch.cuda.synchronize()
    return to_np(C)


GPU = {"w4a4": gpu_w4a4, "w4a8": gpu_w4a8, "w4a16": gpu_w4a16, "bf16": gpu_bf16}


# ----------------------------------------------------------- oracle side
def operands(fmt, inp):
    if fmt == "w4a4":
        return (Operand(NVFP4, inp["aq"], inp["as_"], tscale=float(inp["Sa"])),
                Operand(NVFP4, inp["wq"], inp["ws"], tscale=float(inp["Sw"])))
    if fmt == "w4a8":
        return (Operand(FP8TOK, inp["aq"], rowscale=inp["atok"]),
                Operand(NVFP4, inp["wq"], inp["ws"], tscale=float(inp["Sw"])))
    if fmt == "w4a16":
        return (Operand(BF16, inp["a"]), Operand(NVFP4, inp["wq"], inp["ws"], tscale=float(inp["Sw"])))
    if fmt == "bf16":
        return Operand(BF16, inp["a"]), Operand(BF16, inp["w"])
    raise ValueError(fmt)


def oracle_full(fmt, inp):
    A, W = operands(fmt, inp)
    return oracle.gemm_full(A, W)


def oracle_points(fmt, inp, m, n):
    A, W = operands(fmt, inp)
    return oracle.gemm_points(A, W, m, n)


def w4a8_window(inp, m=None, n=None):
    """FP8 MFMA summation-window allowance (fp8_window_bound) of each W4A8
    output, everywhere [M,N] or at the points (m[i], n[i]).  The MFMA's
    operands are the E4M3 token values and the weight's E2M1 values times
    2^-6 (the E2M1 -> E4M3 identity); a group's sum is then multiplied by 64
    times its E4M3 weight scale, the token factor and the tensor scale."""
    e4 = np.array([oracle.dec_e4m3(b) for b in range(256)])
    e2 = np.array([oracle.dec_e2m1(c) for c in range(16)]) * 2.0 ** -6
    aq, wq, ws = inp["aq"], inp["wq"], inp["ws"]
    M, N = aq.shape[0], wq.shape[0]
    rf = np.asarray(inp["atok"], dtype=np.float64).ravel() * float(np.ravel(inp["Sw"])[0])

    def wvals(rows):                     # converted weight values [rows, K], factor per 8 [rows, K/8]
        q = wq[rows].astype(np.int64)
        codes = np.empty((q.shape[0], 2 * q.shape[1]), np.int64)
        codes[:, 0::2] = q & 15
        codes[:, 1::2] = q >> 4
        return e2[codes], 64.0 * np.repeat(e4[ws[rows].astype(np.int64)], 2, axis=1)

    if m is None:
        wv, gs = wvals(np.arange(N))
        out = np.empty((M, N))
        for i in range(M):
            out[i] = fp8_window_bound(e4[aq[i].astype(np.int64)][None, :], wv, gs) * rf[i]
        return out
    m, n = np.asarray(m).ravel(), np.asarray(n).ravel()
    out = np.empty(m.size)
    for s in range(0, m.size, 256):
        mi, ni = m[s:s + 256], n[s:s + 256]
        wv, gs = wvals(ni)
        out[s:s + 256] = fp8_window_bound(e4[aq[mi].astype(np.int64)], wv, gs) * rf[mi]
    return out


def check_both(fmt, inp, c64, b64, m=None, n=None, what=""):
    """Run the GPU path in FP32 and BF16 output modes and compare both with
    the oracle (at the given points, or everywhere).  W4A8 sums on the FP8
    MFMA, so its tolerance adds that instruction's summation-window
    allowance.  Returns max err/B."""
    g32 = GPU[fmt](inp, True)
    g16 = GPU[fmt](inp, False)
    if m is not None:
        g32, g16 = g32[m, n], g16[m, n]
    extra = w4a8_window(inp, m, n) if fmt == "w4a8" else None
    if fmt == "w4a4":
        check_w4a4_route_exact(inp, g32, g16, m, n, what)
    rel = check_f32(g32, c64, b64, what=what + " fp32", extra=extra)
    loose = check_bf16_vs(g16, c64, b64, what=what + " bf16", extra=extra, g32=g32)
    report(what, g32, c64, b64, extra, loose)
    return rel, g32, g16


def f32_to_bf16_rne(v):
    """BF16 bits of FP32 values, round to nearest even (finite inputs)"""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_w4a4_route_exact(inp, g32, g16, m=None, n=None, what=""):
    """W4A4 bit for bit: every FP32 output equals the oracle's emulation of
    the exact FP8 route (orc_fp8route_w4a4_point: group partials exact,
    fma(c_g, P_g, acc) in FP32, groups ascending) times the FP32 product of
    the tensor scales, rounded once in FP32; every BF16 output is that value
    rounded to nearest even.  (The kernel scales each term and partial sum by
    exactly 2^-12 and puts 4096 into the epilogue factor, which changes no
    rounding.)"""
    M, N = inp["aq"].shape[0], inp["wq"].shape[0]
    if m is None:
        mm, nn = np.divmod(np.arange(M * N, dtype=np.int64), N)
    else:
        mm, nn = np.asarray(m).ravel(), np.asarray(n).ravel()
    route = oracle.fp8route_w4a4_points(inp["aq"], inp["as_"], inp["wq"], inp["ws"], mm, nn)
    gs = np.float32(np.float32(np.ravel(inp["Sa"])[0]) * np.float32(np.ravel(inp["Sw"])[0]))
    want = (route * gs).astype(np.float32)
    got = np.asarray(g32, np.float32).ravel()
    bad = np.where(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} FP32 outputs differ from the route "
                           f"emulation; first {bad[:5]}: gpu {got[bad[:5]]} route {want[bad[:5]]}")
    g16 = np.asarray(g16).ravel().astype(np.uint16)
    bad = np.where(g16 != f32_to_bf16_rne(want))[0]
    assert bad.size == 0, f"{what}: {bad.size} BF16 outputs differ from RNE(route); first {bad[:5]}"
    print(f"[parity] {what}: {got.size} outputs bit-identical to the emulated exact FP8 route")


def report(what, g32, c64, b64, extra=None, loose=0):
    """Print how close an FP32 result came to the bare 1e-5*B tolerance: the
    outputs beyond it (covered by the FP8 window allowance), the largest
    err / (1e-5*B), the largest share of the window allowance used, and the
    BF16 outputs that needed the cancellation rule of check_bf16_vs."""
    err = np.abs(np.asarray(g32, np.float64).ravel() - np.asarray(c64).ravel())
    lim = 1e-5 * np.asarray(b64).ravel()
    nz = lim > 0
    ratio = err[nz] / lim[nz]
    over = int((err > lim).sum())
    line = f"[parity] {what}: {err.size} outputs, max err/(1e-5 B) = {ratio.max() if ratio.size else 0:.3g}"
    if extra is not None:
        ex = np.asarray(extra).ravel()
        use = np.where(ex > 0, np.maximum(err - lim, 0) / np.where(ex > 0, ex, 1), 0)
        line += f", beyond 1e-5 B: {over}, window allowance nonzero at {int((ex > 0).sum())}, " \
                f"max share of it used {use.max():.3g}"
    line += f", BF16 beyond 1 ulp (cancellation rule): {loose}"
    print(line)


def check_bf16_vs(g16, c64, b64, what="", extra=None, g32=None):
    """BF16 output: within 1 BF16 ulp of RNE(oracle).  Where cancellation
    makes the FP32 tolerance 1e-5*B (+ extra) wider than that ulp, a BF16
    output may sit further away only as the rounding of a correct FP32
    result: when the same call's FP32 output g32 is given (checked against
    the FP32 tolerance by the caller), every BF16 output must be exactly
    RNE(g32), and an output beyond 1 ulp must lie within the FP32 tolerance
    of the oracle plus one ulp.  Returns the number of outputs beyond 1 ulp."""
    ref = oracle.bf16_rne(np.asarray(c64).ravel())
    g = np.asarray(g16).ravel()
    from checks import bf16_ordinal
    assert g.size > 0
    if g32 is not None:
        r32 = f32_to_bf16_rne(np.asarray(g32).ravel())
        bad = np.where(g.astype(np.uint16) != r32)[0]
        assert bad.size == 0, f"{what}: {bad.size} BF16 outputs are not RNE of the FP32 result; first {bad[:5]}"
    d = np.abs(bf16_ordinal(g) - bf16_ordinal(ref))
    gv = torch.tensor(g.view(np.int16)).view(torch.bfloat16).double().numpy()
    c = np.asarray(c64).ravel()
    ulp = np.abs(c) * 2.0 ** -8 + 2.0 ** -133
    tol = 1e-5 * np.asarray(b64).ravel()
    if extra is not None:
        tol = tol + np.asarray(extra).ravel()
    loose = (np.abs(gv - c) <= tol + ulp) & (tol > 2.0 ** -9 * np.abs(c))
    bad = np.where((d > 1) & ~loose)[0]
    assert bad.size == 0, f"{what}: {bad.size} BF16 outputs off; first {bad[:5]} gpu {g[bad[:5]]} ref {ref[bad[:5]]}"
    return int((d > 1).sum())
