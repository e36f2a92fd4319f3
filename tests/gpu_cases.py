"""Shared helpers for the GPU parity tests: run each entry point of the HIP
library through the Python binding on given bytes, and compute the oracle's
answer for the same bytes.  Test infrastructure only."""
import numpy as np
import torch

import block_scaled_precision_tn_amd as mg
import oracle
from oracle import BF16, FP8TOK, MXFP8, NVFP4, Operand

from checks import check_bf16, check_f32


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


def check_both(fmt, inp, c64, b64, m=None, n=None, what=""):
    """Run the GPU path in FP32 and BF16 output modes and compare both with
    the oracle (at the given points, or everywhere).  Returns max err/B."""
    g32 = GPU[fmt](inp, True)
    g16 = GPU[fmt](inp, False)
    if m is not None:
        g32, g16 = g32[m, n], g16[m, n]
    rel = check_f32(g32, c64, b64, what=what + " fp32")
    check_bf16_vs(g16, c64, b64, what=what + " bf16")
    return rel, g32, g16


def check_bf16_vs(g16, c64, b64, what="", extra=None):
    """BF16 output: within 1 BF16 ulp of RNE(oracle); where cancellation makes
    the FP32 tolerance 1e-5*B (+ extra) wider than that ulp, within the FP32
    tolerance plus one BF16 ulp instead (the rounding of a correct FP32
    result)."""
    ref = oracle.bf16_rne(np.asarray(c64).ravel())
    g = np.asarray(g16).ravel()
    from checks import bf16_ordinal
    d = np.abs(bf16_ordinal(g) - bf16_ordinal(ref))
    gv = torch.tensor(g.view(np.int16)).view(torch.bfloat16).double().numpy()
    c = np.asarray(c64).ravel()
    ulp = np.abs(c) * 2.0 ** -8 + 2.0 ** -133
    tol = 1e-5 * np.asarray(b64).ravel()
    if extra is not None:
        tol = tol + np.asarray(extra).ravel()
    loose = np.abs(gv - c) <= tol + ulp
    bad = np.where((d > 1) & ~loose)[0]
    assert g.size > 0
    assert bad.size == 0, f"{what}: {bad.size} BF16 outputs off; first {bad[:5]} gpu {g[bad[:5]]} ref {ref[bad[:5]]}"
    return int(((d > 1) & loose).sum())
