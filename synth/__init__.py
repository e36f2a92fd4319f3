"""Seeded synthetic workloads for the block-scaled TN GEMM.

This module only *makes inputs*: random FP32 tensors with the distributions of
the workloads, and their encodings into the declared storage formats (BF16,
NVFP4, FP8 E4M3 with a per-token scale, MXFP8).  It holds no GEMM, decode or
accumulation arithmetic: the oracle under ``oracle/`` and the HIP library each
implement that on their own.  Both consume the bytes made here.

Encodings follow the usual definitions of the formats; the pages only name
them (metrale_circuit ``hardware::exec`` module description for NVFP4 / FP8 /
BF16, the FlashInfer ``swapab_cutedsl_megakernel`` skill page for MXFP8):

* NVFP4: FP32 tensor scale ``S = amax/(448*6)`` (1 if the tensor is zero);
  per 16-element group an E4M3 scale ``RNE(amax_g/6/S)``; E2M1 codes
  ``RNE(x/(scale*S))`` saturating at 6; element ``2i`` in the low nibble.
* FP8 per token: ``s = amax_row/448`` (1 if zero), codes ``RNE_E4M3(a/s)``.
* MXFP8 (OCP MX): per 32-element block ``X = floor(log2 amax) - 8`` clamped
  to [-127, 127], E8M0 byte ``X+127`` (0 for an all-zero block), codes
  ``RNE_E4M3(v/2^X)`` saturating at 448.

Normal samples come from a counter-based generator (SplitMix64 over a key
derived from (seed, tensor role) and the element index, Box-Muller pairs), so
every tensor is reproducible on its own and independent of thread count; the
bulk work runs in ``synth.c`` (multi-threaded C).  The small random choices
(outlier columns, routing logits) use ``numpy.random.default_rng`` streams
spawned from ``SeedSequence(seed)``.  The numpy encoders below (``np_*``) are a
second, independent implementation kept to cross-check the C ones.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared",
                           "-Wall", _SRC, "-o", tmp, "-lm", "-lpthread"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = C.CDLL(_LIB)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    lib.syn_key.restype = C.c_uint64
    lib.syn_key.argtypes = [C.c_uint64, C.c_uint64]
    lib.syn_normal.restype = None
    lib.syn_normal.argtypes = [C.c_uint64, C.c_float, vp, i64, i32]
    lib.syn_quant_nvfp4.restype = C.c_float
    lib.syn_quant_nvfp4.argtypes = [vp, i64, i64, vp, vp, i32]
    lib.syn_quant_fp8_token.restype = None
    lib.syn_quant_fp8_token.argtypes = [vp, i64, i64, vp, vp, i32]
    lib.syn_quant_mxfp8.restype = None
    lib.syn_quant_mxfp8.argtypes = [vp, i64, vp, vp, i32]
    lib.syn_to_bf16.restype = None
    lib.syn_to_bf16.argtypes = [vp, i64, vp, i32]
    _lib = lib
    return lib


def _nth():
    return max(1, min(os.cpu_count() or 1, 16))

# one child stream per tensor role
ROLE_A, ROLE_W, ROLE_OUTLIER, ROLE_LOGITS, ROLE_W2 = 0, 1, 2, 3, 4
_NROLES = 8

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def role_rng(seed: int, role: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(_NROLES)[role])


def normal(shape, std: float, seed: int, role: int) -> np.ndarray:
    """FP32 samples of N(0, std^2) (counter-based, see the module note)."""
    x = np.empty(shape, dtype=np.float32)
    lib = _load()
    lib.syn_normal(lib.syn_key(seed, role), float(std), x.ctypes.data, x.size, _nth())
    return x


def outlier_columns(K: int, seed: int, frac: float = 0.01) -> np.ndarray:
    """floor(frac*K) distinct column indices, drawn without replacement."""
    n = int(np.floor(frac * K))
    return np.sort(role_rng(seed, ROLE_OUTLIER).choice(K, size=n, replace=False))


def with_outliers(a: np.ndarray, cols: np.ndarray, factor: float = 20.0) -> np.ndarray:
    a[:, cols] *= np.float32(factor)
    return a


# ----------------------------------------------------------------- encoders
def np_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 to BF16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def _e4m3_encode(v: np.ndarray) -> np.ndarray:
    """FP64 array -> E4M3-FN bytes, nearest-even, saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)              # exponent of the binade (or subnormal)
    step = np.ldexp(1.0, e - 3)             # 3 mantissa bits
    r = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    _, ex2 = np.frexp(r)
    er = ex2 - 1
    normal = r >= 2.0 ** -6
    mant_n = np.rint((r / np.ldexp(1.0, np.where(normal, er, 0)) - 1.0) * 8.0)
    code_n = ((er + 7) << 3) + mant_n.astype(np.int64)
    code_s = np.rint(r / 2.0 ** -9).astype(np.int64)   # subnormal: m * 2^-9
    code = np.where(normal, code_n, code_s)
    code = np.where(r == 0, 0, code)
    return (code.astype(np.uint8) | sign)


def _e4m3_value(b: np.ndarray) -> np.ndarray:
    """E4M3-FN bytes -> FP64 values (used only to form the encoders' divisors)."""
    b = np.asarray(b, dtype=np.int64)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where(b & 0x80, -v, v)


_E2M1_BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _e2m1_encode(x: np.ndarray) -> np.ndarray:
    """FP64 array -> 4-bit E2M1 codes, nearest with ties to even, saturating."""
    a = np.abs(x)
    # magnitude index on the grid {0,.5,1,1.5,2,3,4,6}; at a tie the even code
    # (mantissa bit 0) wins: bounds that tie to the upper code use side='left'
    lo = np.searchsorted(_E2M1_BOUNDS, a, side="left")
    hi = np.searchsorted(_E2M1_BOUNDS, a, side="right")
    idx = np.where(hi != lo, np.where(lo % 2 == 0, lo, hi), lo)
    return (idx.astype(np.uint8) | np.where(np.signbit(x) & (idx > 0), 8, 0).astype(np.uint8))


def np_quant_nvfp4(x: np.ndarray, chunk_rows: int = 1024):
    """FP32 [R,K] -> (codes uint8 [R,K/2], scales uint8 [R,K/16], S float32)."""
    R, K = x.shape
    assert K % 16 == 0
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    S = np.float32(amax / (E4M3_MAX * E2M1_MAX)) if amax > 0 else np.float32(1.0)
    if S == 0:
        S = np.float32(1.0)
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 16), np.uint8)
    for r0 in range(0, R, chunk_rows):
        xs = x[r0:r0 + chunk_rows].astype(np.float64).reshape(-1, K // 16, 16)
        amax_g = np.abs(xs).max(axis=2)
        sb = _e4m3_encode(amax_g / E2M1_MAX / float(S))
        div = _e4m3_value(sb) * float(S)
        safe = np.where(div == 0, 1.0, div)
        q = np.where(div[..., None] == 0, 0.0, xs / safe[..., None])
        c = _e2m1_encode(q).reshape(xs.shape[0], K)
        codes[r0:r0 + chunk_rows] = c[:, 0::2] | (c[:, 1::2] << 4)
        scales[r0:r0 + chunk_rows] = sb
    return codes, scales, S


def np_quant_fp8_token(a: np.ndarray, chunk_rows: int = 1024):
    """FP32 [M,K] -> (E4M3 bytes [M,K], per-token FP32 scale [M])."""
    M, K = a.shape
    amax = np.abs(a).max(axis=1).astype(np.float32) if K else np.zeros(M, np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = np.empty((M, K), np.uint8)
    for r0 in range(0, M, chunk_rows):
        q[r0:r0 + chunk_rows] = _e4m3_encode(
            a[r0:r0 + chunk_rows].astype(np.float64) / s[r0:r0 + chunk_rows, None].astype(np.float64))
    return q, s


def np_quant_mxfp8(v: np.ndarray, chunk_rows: int = 512):
    """FP32 [..., K] -> (E4M3 bytes [..., K], E8M0 bytes [..., K/32])."""
    shape = v.shape
    K = shape[-1]
    assert K % 32 == 0
    flat = v.reshape(-1, K)
    codes = np.empty(flat.shape, np.uint8)
    scales = np.empty((flat.shape[0], K // 32), np.uint8)
    for r0 in range(0, flat.shape[0], chunk_rows):
        blk = flat[r0:r0 + chunk_rows].astype(np.float64).reshape(-1, K // 32, 32)
        amax = np.abs(blk).max(axis=2)
        _, ex = np.frexp(amax)
        X = np.clip(ex - 1 - 8, -127, 127)
        X = np.where(amax == 0, -127, X)
        scales[r0:r0 + chunk_rows] = (X + 127).astype(np.uint8)
        c = _e4m3_encode(np.ldexp(blk, -X[..., None]))
        codes[r0:r0 + chunk_rows] = c.reshape(-1, K)
    return codes.reshape(shape), scales.reshape(shape[:-1] + (K // 32,))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round FP32 to BF16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().syn_to_bf16(x.ctypes.data, x.size, out.ctypes.data, _nth())
    return out


def quant_nvfp4(x: np.ndarray):
    """FP32 [R,K] -> (codes uint8 [R,K/2], scales uint8 [R,K/16], S float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    assert K % 16 == 0
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 16), np.uint8)
    S = _load().syn_quant_nvfp4(x.ctypes.data, R, K, codes.ctypes.data, scales.ctypes.data, _nth())
    return codes, scales, np.float32(S)


def quant_fp8_token(a: np.ndarray):
    """FP32 [M,K] -> (E4M3 bytes [M,K], per-token FP32 scale [M])."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    M, K = a.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty(M, np.float32)
    _load().syn_quant_fp8_token(a.ctypes.data, M, K, q.ctypes.data, s.ctypes.data, _nth())
    return q, s


def quant_mxfp8(v: np.ndarray):
    """FP32 [..., K] -> (E4M3 bytes [..., K], E8M0 bytes [..., K/32])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    K = v.shape[-1]
    assert K % 32 == 0
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (K // 32,), np.uint8)
    _load().syn_quant_mxfp8(v.ctypes.data, v.size, codes.ctypes.data, scales.ctypes.data, _nth())
    return codes, scales


def topk_routing(T: int, E: int, topk: int, seed: int):
    """Softmax of N(0,1) logits [T,E] in FP64; top-k by probability, ties to the
    lower expert id; weights are the (unrenormalised) probabilities in FP32."""
    logits = role_rng(seed, ROLE_LOGITS).standard_normal(size=(T, E))
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :topk].astype(np.int32)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(np.float32)
    return ids, w


# --------------------------------------------------------------- workloads
def w4a16(M, N, K, seed=0, w_std=0.02, a_outliers=False):
    a = normal((M, K), 1.0, seed, ROLE_A)
    if a_outliers:
        with_outliers(a, outlier_columns(K, seed))
    w = normal((N, K), w_std, seed, ROLE_W)
    wq, ws, Sw = quant_nvfp4(w)
    return dict(a=to_bf16_bits(a), wq=wq, ws=ws, Sw=Sw)


def bf16(M, N, K, seed=0, a_outliers=True):
    a = normal((M, K), 1.0, seed, ROLE_A)
    if a_outliers:
        with_outliers(a, outlier_columns(K, seed))
    w = normal((N, K), 1.0 / np.sqrt(K), seed, ROLE_W)
    return dict(a=to_bf16_bits(a), w=to_bf16_bits(w))


def w4a4(M, N, K, seed=0, w_std=0.02, a_outliers=True):
    a = normal((M, K), 1.0, seed, ROLE_A)
    if a_outliers:
        with_outliers(a, outlier_columns(K, seed))
    aq, as_, Sa = quant_nvfp4(a)
    del a
    w = normal((N, K), w_std, seed, ROLE_W)
    wq, ws, Sw = quant_nvfp4(w)
    return dict(aq=aq, as_=as_, Sa=Sa, wq=wq, ws=ws, Sw=Sw)


def w4a8(M, N, K, seed=0, w_std=0.02):
    a = normal((M, K), 1.0, seed, ROLE_A)
    aq, atok = quant_fp8_token(a)
    w = normal((N, K), w_std, seed, ROLE_W)
    wq, ws, Sw = quant_nvfp4(w)
    return dict(aq=aq, atok=atok, wq=wq, ws=ws, Sw=Sw)


def moe(T, H, I, E, topk, seed=0, w_std=0.02):
    x = normal((T, H), 1.0, seed, ROLE_A)
    xq, xs = quant_mxfp8(x)
    del x
    w13 = normal((E, 2 * I, H), w_std, seed, ROLE_W)
    w13q, w13s = quant_mxfp8(w13)
    del w13
    w2 = normal((E, H, I), w_std, seed, ROLE_W2)
    w2q, w2s = quant_mxfp8(w2)
    del w2
    ids, tw = topk_routing(T, E, topk, seed)
    return dict(xq=xq, xs=xs, w13q=w13q, w13s=w13s, w2q=w2q, w2s=w2s, ids=ids, tw=tw)


# static tensor scale of the NVFP4 re-quantisation of h in the NVFP4 MoE
# (the caller fixes it; 2^-8 puts the group scales amax / 6 / S_h of the
# workload's h, |h| within about 2^-7 .. 2^4, inside the E4M3 range)
MOE4_SH = 2.0 ** -8


def moe_nvfp4(T, H, I, E, topk, seed=0, w_std=0.02):
    """NVFP4 MoE inputs: x ~ N(0,1) and the experts' w13, w2 ~ N(0, w_std)
    quantised to NVFP4 (x with one tensor scale, each expert's matrices with
    their own), the same routing as moe()."""
    x = normal((T, H), 1.0, seed, ROLE_A)
    xq, xs, Sx = quant_nvfp4(x)
    del x
    w13q = np.empty((E, 2 * I, H // 2), np.uint8)
    w13s = np.empty((E, 2 * I, H // 16), np.uint8)
    w2q = np.empty((E, H, I // 2), np.uint8)
    w2s = np.empty((E, H, I // 16), np.uint8)
    Sw13 = np.empty(E, np.float32)
    Sw2 = np.empty(E, np.float32)
    w13 = normal((E, 2 * I, H), w_std, seed, ROLE_W)
    for e in range(E):
        w13q[e], w13s[e], Sw13[e] = quant_nvfp4(w13[e])
    del w13
    w2 = normal((E, H, I), w_std, seed, ROLE_W2)
    for e in range(E):
        w2q[e], w2s[e], Sw2[e] = quant_nvfp4(w2[e])
    del w2
    ids, tw = topk_routing(T, E, topk, seed)
    return dict(xq=xq, xs=xs, Sx=Sx, w13q=w13q, w13s=w13s, Sw13=Sw13, w2q=w2q, w2s=w2s, Sw2=Sw2,
                Sh=np.float32(MOE4_SH), ids=ids, tw=tw)


def moe_logits(T: int, E: int, seed: int = 0) -> np.ndarray:
    """Router logits [T,E] ~N(0,1) in FP32 (the draw topk_routing uses)."""
    return role_rng(seed, ROLE_LOGITS).standard_normal(size=(T, E)).astype(np.float32)
