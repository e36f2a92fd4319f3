"""Python access to the plain FP64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the product (the HIP library and its
binding) never imports it.  The oracle shares no code with the GPU path.

``build()`` compiles ``oracle.c`` with gcc into ``liboracle.so`` beside it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, NVFP4, FP8TOK, MXFP8 = 0, 1, 2, 3


def build() -> str:
    """Compile the oracle (plain C, no fast-math)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared",
                           "-Wall", _SRC, "-o", tmp, "-lm", "-lpthread"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = C.CDLL(_LIB_PATH)
    i64, f64, u8p = C.c_int64, C.c_double, C.POINTER(C.c_uint8)
    lib.orc_dec_bf16.restype = f64
    lib.orc_dec_bf16.argtypes = [C.c_uint16]
    for n in ("orc_dec_e2m1", "orc_dec_e4m3", "orc_dec_e8m0"):
        getattr(lib, n).restype = f64
        getattr(lib, n).argtypes = [C.c_uint8]
    lib.orc_gemm_points.restype = C.c_int
    lib.orc_gemm_points.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, i64,
                                    C.c_void_p, C.c_void_p, C.c_int]
    lib.orc_gemm_full.restype = C.c_int
    lib.orc_gemm_full.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int]
    lib.orc_fp8route_convert_word.restype = C.c_uint32
    lib.orc_fp8route_convert_word.argtypes = [C.c_uint32]
    lib.orc_fp8route_w4a4_point.restype = C.c_float
    lib.orc_fp8route_w4a4_point.argtypes = [C.c_void_p] * 4 + [i64]
    lib.orc_fp8route_w4a8_point.restype = C.c_float
    lib.orc_fp8route_w4a8_point.argtypes = [C.c_void_p] * 3 + [i64]
    lib.orc_fp8route_w4a4_rows.restype = None
    lib.orc_fp8route_w4a4_rows.argtypes = [C.c_void_p] * 4 + [i64, i64, C.c_void_p]
    lib.orc_fp8route_w4a8_rows.restype = None
    lib.orc_fp8route_w4a8_rows.argtypes = [C.c_void_p] * 3 + [i64, i64, C.c_void_p]
    lib.orc_fp8route_w4a4_points.restype = C.c_int
    lib.orc_fp8route_w4a4_points.argtypes = [C.c_void_p] * 4 + [i64] * 3 + [C.c_void_p] * 2 + \
        [i64, C.c_void_p, C.c_int]
    lib.orc_enc_e4m3_rne_sat.restype = C.c_uint8
    lib.orc_enc_e4m3_rne_sat.argtypes = [f64]
    lib.orc_mxq.restype = None
    lib.orc_mxq.argtypes = [C.c_void_p, i64, C.c_void_p, C.c_void_p]
    lib.orc_bf16_rne.restype = C.c_uint16
    lib.orc_bf16_rne.argtypes = [f64]
    lib.orc_moe_gateup.restype = None
    lib.orc_moe_gateup.argtypes = [C.c_void_p, C.c_void_p, i64, i64, C.c_void_p, C.c_void_p,
                                   i64, i64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.orc_moe_glu_requant.restype = None
    lib.orc_moe_glu_requant.argtypes = [C.c_void_p, C.c_void_p, i64, C.c_void_p, C.c_void_p]
    lib.orc_moe_down.restype = None
    lib.orc_moe_down.argtypes = [C.c_void_p, C.c_void_p, i64, C.c_void_p, C.c_void_p, i64, i64,
                                 C.c_void_p, C.c_void_p]
    lib.orc_moe_tokens.restype = C.c_int
    lib.orc_moe_tokens.argtypes = [C.c_void_p] * 4 + [i64] * 5 + [C.c_void_p] * 5 + [i64] + \
        [C.c_void_p, C.c_void_p, C.c_int]
    f32 = C.c_float
    lib.orc_enc_e2m1_rne_sat.restype = C.c_uint8
    lib.orc_enc_e2m1_rne_sat.argtypes = [f32]
    lib.orc_nvq.restype = None
    lib.orc_nvq.argtypes = [C.c_void_p, i64, f32, C.c_void_p, C.c_void_p]
    lib.orc_moe4_gateup.restype = None
    lib.orc_moe4_gateup.argtypes = [C.c_void_p, C.c_void_p, f32, i64, i64, C.c_void_p,
                                    C.c_void_p, C.c_void_p, i64, i64] + [C.c_void_p] * 4
    lib.orc_moe4_glu_requant.restype = None
    lib.orc_moe4_glu_requant.argtypes = [C.c_void_p, C.c_void_p, i64, f32, C.c_void_p,
                                         C.c_void_p]
    lib.orc_moe4_down.restype = None
    lib.orc_moe4_down.argtypes = [C.c_void_p, C.c_void_p, f32, i64, C.c_void_p, C.c_void_p,
                                  C.c_void_p, i64, i64, C.c_void_p, C.c_void_p]
    lib.orc_moe4_tokens.restype = C.c_int
    lib.orc_moe4_tokens.argtypes = [C.c_void_p, C.c_void_p, f32, C.c_void_p, C.c_void_p] + \
        [i64] * 5 + [C.c_void_p] * 6 + [f32, C.c_void_p, i64, C.c_void_p, C.c_void_p, C.c_int]
    lib.orc_topk_softmax.restype = C.c_int
    lib.orc_topk_softmax.argtypes = [C.c_void_p, i64, i64, i64, C.c_void_p, C.c_void_p]
    _lib = lib
    return lib


class _Operand(C.Structure):
    _fields_ = [("fmt", C.c_int), ("data", C.c_void_p), ("scales", C.c_void_p),
                ("rowscale", C.c_void_p), ("tscale", C.c_double), ("R", C.c_int64),
                ("K", C.c_int64)]


@dataclass
class Operand:
    """An operand in a declared storage format (numpy arrays, C-contiguous)."""
    fmt: int
    data: np.ndarray
    scales: Optional[np.ndarray] = None
    rowscale: Optional[np.ndarray] = None
    tscale: float = 1.0

    @property
    def R(self) -> int:
        return self.data.shape[0]

    @property
    def K(self) -> int:
        return self.data.shape[1] * (2 if self.fmt == NVFP4 else 1)

    def _c(self):
        keep = [np.ascontiguousarray(self.data)]
        ptr = lambda a: a.ctypes.data if a is not None else None  # noqa: E731
        sc = None if self.scales is None else np.ascontiguousarray(self.scales, dtype=np.uint8)
        rs = None if self.rowscale is None else np.ascontiguousarray(self.rowscale, dtype=np.float32)
        keep += [sc, rs]
        return _Operand(self.fmt, ptr(keep[0]), ptr(sc), ptr(rs), float(self.tscale),
                        self.R, self.K), keep


def _nthreads(n):
    return int(n) if n else (os.cpu_count() or 1)


def dec_bf16(u):
    return _load().orc_dec_bf16(int(u))


def dec_e2m1(c):
    return _load().orc_dec_e2m1(int(c))


def dec_e4m3(b):
    return _load().orc_dec_e4m3(int(b))


def dec_e8m0(x):
    return _load().orc_dec_e8m0(int(x))


def elem_values(op: Operand) -> np.ndarray:
    """Decoded element values (block scales included, row factors not), FP64
    [R,K].  Built from the scalar decoders; for small operands only."""
    lib = _load()
    R, K = op.R, op.K
    out = np.empty((R, K))
    if op.fmt == BF16:
        lut = np.array([lib.orc_dec_bf16(u) for u in range(65536)])
        return lut[op.data.astype(np.int64)]
    e4 = np.array([lib.orc_dec_e4m3(b) for b in range(256)])
    if op.fmt == NVFP4:
        e2 = np.array([lib.orc_dec_e2m1(c) for c in range(16)])
        codes = np.empty((R, K), np.int64)
        codes[:, 0::2] = op.data & 15
        codes[:, 1::2] = op.data >> 4
        sc = np.repeat(e4[op.scales.astype(np.int64)], 16, axis=1)
        out[:] = e2[codes] * sc
    elif op.fmt == FP8TOK:
        out[:] = e4[op.data.astype(np.int64)]
    else:
        e8 = np.array([lib.orc_dec_e8m0(x) for x in range(256)])
        out[:] = e4[op.data.astype(np.int64)] * np.repeat(e8[op.scales.astype(np.int64)], 32, axis=1)
    return out


def gemm_points(A: Operand, W: Operand, m, n, nthreads=None):
    """(C, B) in FP64 at the points (m[i], n[i])."""
    lib = _load()
    m = np.ascontiguousarray(m, dtype=np.int64)
    n = np.ascontiguousarray(n, dtype=np.int64)
    Cv = np.zeros(len(m))
    Bv = np.zeros(len(m))
    ca, ka = A._c()
    cw, kw = W._c()
    rc = lib.orc_gemm_points(C.byref(ca), C.byref(cw), m.ctypes.data, n.ctypes.data, len(m),
                             Cv.ctypes.data, Bv.ctypes.data, _nthreads(nthreads))
    if rc != 0:
        raise ValueError("oracle: bad gemm_points arguments")
    return Cv, Bv


def gemm_full(A: Operand, W: Operand, nthreads=None):
    """(C, B) in FP64, [M,N]."""
    lib = _load()
    Cv = np.zeros((A.R, W.R))
    Bv = np.zeros((A.R, W.R))
    ca, ka = A._c()
    cw, kw = W._c()
    rc = lib.orc_gemm_full(C.byref(ca), C.byref(cw), Cv.ctypes.data, Bv.ctypes.data,
                           _nthreads(nthreads))
    if rc != 0:
        raise ValueError("oracle: bad gemm_full arguments")
    return Cv, Bv


def fp8route_convert_word(q: int) -> int:
    return _load().orc_fp8route_convert_word(q & 0xFFFFFFFF)


def fp8route_w4a4_point(aq, as_, wq, ws) -> float:
    aq, as_, wq, ws = (np.ascontiguousarray(x, dtype=np.uint8) for x in (aq, as_, wq, ws))
    return _load().orc_fp8route_w4a4_point(aq.ctypes.data, as_.ctypes.data, wq.ctypes.data,
                                           ws.ctypes.data, aq.size * 2)


def fp8route_w4a8_point(a8, wq, ws) -> float:
    a8, wq, ws = (np.ascontiguousarray(x, dtype=np.uint8) for x in (a8, wq, ws))
    return _load().orc_fp8route_w4a8_point(a8.ctypes.data, wq.ctypes.data, ws.ctypes.data, a8.size)


def fp8route_w4a4_rows(aq, as_, wq, ws) -> np.ndarray:
    """Emulated exact-FP8 route, row i of A against row i of W."""
    aq, as_, wq, ws = (np.ascontiguousarray(x, dtype=np.uint8) for x in (aq, as_, wq, ws))
    out = np.zeros(aq.shape[0], np.float32)
    _load().orc_fp8route_w4a4_rows(aq.ctypes.data, as_.ctypes.data, wq.ctypes.data,
                                   ws.ctypes.data, aq.shape[1] * 2, aq.shape[0], out.ctypes.data)
    return out


def fp8route_w4a4_points(aq, as_, wq, ws, m, n, nthreads=None) -> np.ndarray:
    """Emulated exact-FP8 route (FP32, before the tensor scales) at the points
    (m[i], n[i]): row m[i] of A against row n[i] of W."""
    aq, as_, wq, ws = (np.ascontiguousarray(x, dtype=np.uint8) for x in (aq, as_, wq, ws))
    m = np.ascontiguousarray(m, dtype=np.int64).ravel()
    n = np.ascontiguousarray(n, dtype=np.int64).ravel()
    out = np.zeros(m.size, np.float32)
    rc = _load().orc_fp8route_w4a4_points(aq.ctypes.data, as_.ctypes.data, wq.ctypes.data,
                                          ws.ctypes.data, aq.shape[0], wq.shape[0],
                                          aq.shape[1] * 2, m.ctypes.data, n.ctypes.data, m.size,
                                          out.ctypes.data, _nthreads(nthreads))
    if rc != 0:
        raise ValueError("oracle: bad fp8route points arguments")
    return out


def fp8route_w4a8_rows(a8, wq, ws) -> np.ndarray:
    a8, wq, ws = (np.ascontiguousarray(x, dtype=np.uint8) for x in (a8, wq, ws))
    out = np.zeros(a8.shape[0], np.float32)
    _load().orc_fp8route_w4a8_rows(a8.ctypes.data, wq.ctypes.data, ws.ctypes.data,
                                   a8.shape[1], a8.shape[0], out.ctypes.data)
    return out


def enc_e4m3(v: float) -> int:
    return _load().orc_enc_e4m3_rne_sat(float(v))


def mxq(v):
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    codes = np.zeros(v.size, np.uint8)
    scales = np.zeros(v.size // 32, np.uint8)
    _load().orc_mxq(v.ctypes.data, v.size, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def bf16_rne(v) -> np.ndarray:
    lib = _load()
    v = np.asarray(v, dtype=np.float64)
    return np.array([lib.orc_bf16_rne(float(x)) for x in v.ravel()], dtype=np.uint16).reshape(v.shape)


def moe_gateup(xq, xs, t, e, w13q, w13s, H, I):
    g, u, bg, bu = (np.zeros(I) for _ in range(4))
    _load().orc_moe_gateup(xq.ctypes.data, xs.ctypes.data, t, e, w13q.ctypes.data,
                           w13s.ctypes.data, H, I, g.ctypes.data, u.ctypes.data,
                           bg.ctypes.data, bu.ctypes.data)
    return g, u, bg, bu


def moe_glu_requant(g, u):
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    I = g.size
    hq = np.zeros(I, np.uint8)
    hs = np.zeros(I // 32, np.uint8)
    _load().orc_moe_glu_requant(g.ctypes.data, u.ctypes.data, I, hq.ctypes.data, hs.ctypes.data)
    return hq, hs


def moe_down(hq, hs, e, w2q, w2s, H, I):
    y = np.zeros(H)
    by = np.zeros(H)
    hq = np.ascontiguousarray(hq, dtype=np.uint8)
    hs = np.ascontiguousarray(hs, dtype=np.uint8)
    _load().orc_moe_down(hq.ctypes.data, hs.ctypes.data, e, w2q.ctypes.data, w2s.ctypes.data,
                         H, I, y.ctypes.data, by.ctypes.data)
    return y, by


def moe_tokens(inp: dict, T, H, I, E, topk, tokens, nthreads=None):
    """End-to-end MoE output (FP64) and bound for the listed tokens: [len, H]."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    out = np.zeros((tokens.size, H))
    bound = np.zeros((tokens.size, H))
    a = {k: np.ascontiguousarray(v) for k, v in inp.items()}
    rc = _load().orc_moe_tokens(a["xq"].ctypes.data, a["xs"].ctypes.data, a["ids"].ctypes.data,
                                a["tw"].ctypes.data, T, H, I, E, topk,
                                a["w13q"].ctypes.data, a["w13s"].ctypes.data,
                                a["w2q"].ctypes.data, a["w2s"].ctypes.data,
                                tokens.ctypes.data, tokens.size, out.ctypes.data,
                                bound.ctypes.data, _nthreads(nthreads))
    if rc != 0:
        raise ValueError("oracle: bad moe arguments")
    return out, bound


# ------------------------------------------------------------ NVFP4 MoE
def enc_e2m1(v: float) -> int:
    return _load().orc_enc_e2m1_rne_sat(float(v))


def nvq(v, S):
    """NVFP4 quantisation taken in FP32 under tensor scale S: (codes [n/2], scales [n/16])."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    codes = np.zeros(v.size // 2, np.uint8)
    scales = np.zeros(v.size // 16, np.uint8)
    _load().orc_nvq(v.ctypes.data, v.size, float(S), codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def moe4_gateup(inp, t, e, H, I):
    g, u, bg, bu = (np.zeros(I) for _ in range(4))
    a = {k: np.ascontiguousarray(inp[k]) for k in ("xq", "xs", "w13q", "w13s", "Sw13")}
    _load().orc_moe4_gateup(a["xq"].ctypes.data, a["xs"].ctypes.data, float(inp["Sx"]), t, e,
                            a["w13q"].ctypes.data, a["w13s"].ctypes.data,
                            np.ascontiguousarray(a["Sw13"], np.float32).ctypes.data, H, I,
                            g.ctypes.data, u.ctypes.data, bg.ctypes.data, bu.ctypes.data)
    return g, u, bg, bu


def moe4_glu_requant(g, u, Sh):
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    I = g.size
    hq = np.zeros(I // 2, np.uint8)
    hs = np.zeros(I // 16, np.uint8)
    _load().orc_moe4_glu_requant(g.ctypes.data, u.ctypes.data, I, float(Sh), hq.ctypes.data,
                                 hs.ctypes.data)
    return hq, hs


def moe4_down(hq, hs, Sh, e, inp, H, I):
    y = np.zeros(H)
    by = np.zeros(H)
    hq = np.ascontiguousarray(hq, dtype=np.uint8)
    hs = np.ascontiguousarray(hs, dtype=np.uint8)
    w2q, w2s = np.ascontiguousarray(inp["w2q"]), np.ascontiguousarray(inp["w2s"])
    Sw2 = np.ascontiguousarray(inp["Sw2"], np.float32)
    _load().orc_moe4_down(hq.ctypes.data, hs.ctypes.data, float(Sh), e, w2q.ctypes.data,
                          w2s.ctypes.data, Sw2.ctypes.data, H, I, y.ctypes.data, by.ctypes.data)
    return y, by


def moe4_tokens(inp: dict, T, H, I, E, topk, tokens, nthreads=None):
    """End-to-end NVFP4 MoE output (FP64) and bound for the listed tokens."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    out = np.zeros((tokens.size, H))
    bound = np.zeros((tokens.size, H))
    a = {k: np.ascontiguousarray(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    Sw13 = np.ascontiguousarray(inp["Sw13"], np.float32)
    Sw2 = np.ascontiguousarray(inp["Sw2"], np.float32)
    rc = _load().orc_moe4_tokens(a["xq"].ctypes.data, a["xs"].ctypes.data, float(inp["Sx"]),
                                 a["ids"].ctypes.data, a["tw"].ctypes.data, T, H, I, E, topk,
                                 a["w13q"].ctypes.data, a["w13s"].ctypes.data, Sw13.ctypes.data,
                                 a["w2q"].ctypes.data, a["w2s"].ctypes.data, Sw2.ctypes.data,
                                 float(inp["Sh"]), tokens.ctypes.data, tokens.size,
                                 out.ctypes.data, bound.ctypes.data, _nthreads(nthreads))
    if rc != 0:
        raise ValueError("oracle: bad moe4 arguments")
    return out, bound


# ---------------------------------------------------------- top-k routing
def topk_softmax(logits, topk):
    """(ids int32 [T,topk], weights float32 [T,topk]) of FP32 logits [T,E]."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.zeros((T, topk), np.int32)
    w = np.zeros((T, topk), np.float32)
    if _load().orc_topk_softmax(lg.ctypes.data, T, E, topk, ids.ctypes.data, w.ctypes.data) != 0:
        raise ValueError("oracle: bad routing arguments")
    return ids, w
