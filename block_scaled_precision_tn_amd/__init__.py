"""Python binding of libmgemm (the gfx950 block-scaled TN GEMM library).

Argument marshalling only: every function here checks tensor dtypes, shapes,
devices and contiguity, then calls the C entry point of the same name in
``libmgemm.so`` with raw device pointers and the current HIP stream.  All
arithmetic runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, importing works but every call raises.

Tensors are torch tensors on the current GPU, C-contiguous:

  BF16 operands      torch.bfloat16 (or uint16/int16 bit patterns) [R, K]
  NVFP4 codes        torch.uint8 [R, K/2]  (element 2i in the low nibble)
  NVFP4 scales       torch.uint8 [R, K/16] (E4M3-FN bytes)
  FP32 tensor scale  torch.float32, one element, on the device
  FP8 activations    torch.uint8 [M, K] (E4M3-FN bytes) + torch.float32 [M]
  MXFP8              torch.uint8 codes [.., K] + torch.uint8 E8M0 [.., K/32]
  C                  torch.bfloat16 [M, N] (BF16 output) or torch.float32
                     [M, N] (the FP32 result after the global scales)
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmgemm.so")

FMT_BF16, FMT_NVFP4, FMT_FP8_E4M3_TOKEN, FMT_MXFP8 = 0, 1, 2, 3
EXEC_NATIVE, EXEC_FP8_EXACT, EXEC_NOPATH = 0, 1, 2
MMA_NONE, MMA_BF16, MMA_FP8, MMA_MX_F8F6F4 = 0, 1, 2, 3
OP_BF16, OP_W4A16, OP_W4A8, OP_W4A4, OP_MOE, OP_MOE_NVFP4 = 0, 1, 2, 3, 4, 5
OP_BF16_DGRAD, OP_BF16_WGRAD = 6, 7

EXEC_NAMES = {EXEC_NATIVE: "native", EXEC_FP8_EXACT: "fp8_exact", EXEC_NOPATH: "nopath"}
MMA_NAMES = {MMA_NONE: "none", MMA_BF16: "bf16", MMA_FP8: "fp8", MMA_MX_F8F6F4: "mx_f8f6f4"}
REASON_NAMES = {0: "none", 1: "no_instruction", 2: "no_kernel", 3: "no_nvfp4_blockscale_mma",
                4: "no_single_mma", 5: "unsupported_device"}


class MgemmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class _Plan(C.Structure):
    _fields_ = [("kind", C.c_int), ("mma", C.c_int), ("reason", C.c_int)]


_lib = None


def load() -> C.CDLL:
    """Load libmgemm.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmgemm.so not found at {LIB_PATH}: build it with "
                           "`python -m block_scaled_precision_tn_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    sig = {
        "mgemm_plan": (i32, [i32, i32, i32, C.POINTER(_Plan)]),
        "mgemm_plan_arch": (i32, [C.c_char_p, i32, i32, C.POINTER(_Plan)]),
        "mgemm_pair_name": (i32, [i32, i32, C.c_char_p, C.c_size_t]),
        "mgemm_bf16": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, C.c_size_t, vp]),
        "mgemm_w4a16": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, C.c_size_t, vp]),
        "mgemm_w4a8": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, C.c_size_t, vp]),
        "mgemm_w4a8_noalloc": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]),
        "mgemm_w4a4": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]),
        "mgemm_moe_mxfp8_glu": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                      vp, vp, C.c_size_t, vp, vp]),
        "mgemm_moe_mxfp8_glu_debug": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                            vp, vp, vp, C.c_size_t, vp, vp, vp]),
        "mgemm_moe_mxfp8_glu_logits": (i32, [vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp,
                                             vp, vp, vp, vp, C.c_size_t, vp, vp]),
        "mgemm_moe_nvfp4_glu": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, C.c_size_t, vp, vp]),
        "mgemm_moe_route_topk": (i32, [vp, i64, i64, i64, vp, vp, vp]),
        "mgemm_bf16_dgrad": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, C.c_size_t, vp]),
        "mgemm_bf16_wgrad": (i32, [vp, vp, vp, i64, i64, i64, i32, vp, C.c_size_t, vp]),
        "mgemm_workspace_bytes": (C.c_size_t, [i32, i64, i64, i64, i64, i64, i64, i64, i64]),
        "mgemm_status_string": (C.c_char_p, [i32]),
        "mgemm_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def available() -> bool:
    return os.path.exists(LIB_PATH)


def status_string(status: int) -> str:
    return load().mgemm_status_string(int(status)).decode()


def version() -> str:
    return load().mgemm_version().decode()


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MgemmError(fn, rc)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtypes, shape=None, numel=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements")


_BF16_T = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)
_U8 = (torch.uint8,)
_F32 = (torch.float32,)
_C_T = (torch.bfloat16, torch.float32)


def _out_f32(c: torch.Tensor) -> int:
    return 1 if c.dtype == torch.float32 else 0


# ------------------------------------------------------------------ planning
def mgemm_plan(device: int, w_fmt: int, a_fmt: int):
    """(kind, mma, reason) for a weight/activation format pair on a device."""
    p = _Plan()
    _check("mgemm_plan", load().mgemm_plan(int(device), int(w_fmt), int(a_fmt), C.byref(p)))
    return p.kind, p.mma, p.reason


def mgemm_plan_arch(arch: str, w_fmt: int, a_fmt: int):
    p = _Plan()
    _check("mgemm_plan_arch", load().mgemm_plan_arch(arch.encode(), int(w_fmt), int(a_fmt),
                                                     C.byref(p)))
    return p.kind, p.mma, p.reason


def mgemm_pair_name(w_fmt: int, a_fmt: int) -> str:
    buf = C.create_string_buffer(16)
    n = load().mgemm_pair_name(int(w_fmt), int(a_fmt), buf, 16)
    if n < 0:
        raise MgemmError("mgemm_pair_name", n)
    return buf.value.decode()


def mgemm_workspace_bytes(op: int, M=0, N=0, K=0, T=0, H=0, I=0, E=0, topk=0) -> int:
    return int(load().mgemm_workspace_bytes(op, M, N, K, T, H, I, E, topk))


# --------------------------------------------------------------------- GEMMs
def mgemm_bf16(A: torch.Tensor, W: torch.Tensor, C_out: torch.Tensor,
               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    M, K = A.shape
    N = W.shape[0]
    _need(A, "A", _BF16_T, (M, K))
    _need(W, "W", _BF16_T, (N, K))
    _need(C_out, "C", _C_T, (M, N))
    need = mgemm_workspace_bytes(OP_BF16, M, N, K)
    if ws is None:
        ws = workspace(need, "bf16", stream)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        raise ValueError("bf16: workspace too small")
    wp = ws.data_ptr() if ws is not None else None
    wb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("mgemm_bf16", load().mgemm_bf16(A.data_ptr(), W.data_ptr(), C_out.data_ptr(), M, N, K,
                                           _out_f32(C_out), wp, wb, _stream(stream)))
    return C_out


def mgemm_w4a16(A, Wq, Ws, Sw, C_out, ws: Optional[torch.Tensor] = None, stream=None):
    M, K = A.shape
    N = Wq.shape[0]
    _need(A, "A", _BF16_T, (M, K))
    _need(Wq, "Wq", _U8, (N, K // 2))
    _need(Ws, "Ws", _U8, (N, K // 16))
    _need(Sw, "Sw", _F32, numel=1)
    _need(C_out, "C", _C_T, (M, N))
    need = mgemm_workspace_bytes(OP_W4A16, M, N, K)
    if ws is None:
        ws = workspace(need, "w4a16", stream)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        raise ValueError("w4a16: workspace too small")
    wp = ws.data_ptr() if ws is not None else None
    wb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("mgemm_w4a16", load().mgemm_w4a16(A.data_ptr(), Wq.data_ptr(), Ws.data_ptr(),
                                             Sw.data_ptr(), C_out.data_ptr(), M, N, K,
                                             _out_f32(C_out), wp, wb, _stream(stream)))
    return C_out


_WS_CACHE = {}


def workspace(nbytes: int, key=None, stream=None) -> Optional[torch.Tensor]:
    """A device workspace of at least nbytes for work enqueued on `stream`
    (None: the current stream), cached per (device, stream, key) and grown on
    demand, so calls on different streams never share one.  The tensor is
    marked as used by that stream: when a larger one replaces it, its memory
    is not handed out again before the work already enqueued there is done."""
    if nbytes == 0:
        return None
    dev = torch.cuda.current_device()
    h = _stream(stream)
    k = (dev, h, key)
    t = _WS_CACHE.get(k)
    if t is None or t.numel() < nbytes:
        t = torch.empty(nbytes, dtype=torch.uint8, device=f"cuda:{dev}")
        if h != torch.cuda.current_stream().cuda_stream:
            t.record_stream(torch.cuda.ExternalStream(h))
        _WS_CACHE[k] = t
    return t


def mgemm_w4a8(Aq, a_tok, Wq, Ws, Sw, C_out, ws: Optional[torch.Tensor] = None, stream=None):
    M, K = Aq.shape
    N = Wq.shape[0]
    _need(Aq, "Aq", _U8, (M, K))
    _need(a_tok, "a_tok", _F32, numel=M)
    _need(Wq, "Wq", _U8, (N, K // 2))
    _need(Ws, "Ws", _U8, (N, K // 16))
    _need(Sw, "Sw", _F32, numel=1)
    _need(C_out, "C", _C_T, (M, N))
    need = mgemm_workspace_bytes(OP_W4A8, M, N, K)
    if ws is None:
        ws = workspace(need, "w4a8", stream)
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        raise ValueError("w4a8: workspace too small")
    wp = ws.data_ptr() if ws is not None else None
    wb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("mgemm_w4a8", load().mgemm_w4a8(Aq.data_ptr(), a_tok.data_ptr(), Wq.data_ptr(),
                                           Ws.data_ptr(), Sw.data_ptr(), C_out.data_ptr(), M, N, K,
                                           _out_f32(C_out), wp, wb, _stream(stream)))
    return C_out


W4A8_NOALLOC_MAX_WS = 48 << 20   # MGEMM_W4A8_NOALLOC_MAX_WS


def mgemm_w4a8_noalloc(Aq, a_tok, Wq, Ws, Sw, C_out, stream=None):
    """mgemm_w4a8 with the split-K partials in the library's fixed per-device
    buffer: allocates nothing (for graph capture and allocation-free loops).
    Calls that overlap on one GPU share that buffer and must be ordered."""
    M, K = Aq.shape
    N = Wq.shape[0]
    _need(Aq, "Aq", _U8, (M, K))
    _need(a_tok, "a_tok", _F32, numel=M)
    _need(Wq, "Wq", _U8, (N, K // 2))
    _need(Ws, "Ws", _U8, (N, K // 16))
    _need(Sw, "Sw", _F32, numel=1)
    _need(C_out, "C", _C_T, (M, N))
    _check("mgemm_w4a8_noalloc", load().mgemm_w4a8_noalloc(
        Aq.data_ptr(), a_tok.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), Sw.data_ptr(),
        C_out.data_ptr(), M, N, K, _out_f32(C_out), _stream(stream)))
    return C_out


def mgemm_w4a4(Aq, As, Sa, Wq, Ws, Sw, C_out, stream=None):
    M = Aq.shape[0]
    K = Aq.shape[1] * 2
    N = Wq.shape[0]
    _need(Aq, "Aq", _U8, (M, K // 2))
    _need(As, "As", _U8, (M, K // 16))
    _need(Sa, "Sa", _F32, numel=1)
    _need(Wq, "Wq", _U8, (N, K // 2))
    _need(Ws, "Ws", _U8, (N, K // 16))
    _need(Sw, "Sw", _F32, numel=1)
    _need(C_out, "C", _C_T, (M, N))
    _check("mgemm_w4a4", load().mgemm_w4a4(Aq.data_ptr(), As.data_ptr(), Sa.data_ptr(),
                                           Wq.data_ptr(), Ws.data_ptr(), Sw.data_ptr(),
                                           C_out.data_ptr(), M, N, K, _out_f32(C_out),
                                           _stream(stream)))
    return C_out


def mgemm_moe_mxfp8_glu(xq, xs, topk_ids, topk_w, w13q, w13s, w2q, w2s, out,
                        ws: Optional[torch.Tensor] = None, dbg_h: Optional[torch.Tensor] = None,
                        stream=None, dbg_gu: Optional[torch.Tensor] = None):
    """The MXFP8 MoE GLU.  dbg_h / dbg_gu: optional taps (uint8 [T*topk*(I +
    I/32)], FP32 [T*topk*2I]); with dbg_gu the call goes through
    mgemm_moe_mxfp8_glu_debug."""
    T, H = xq.shape
    topk = topk_ids.shape[1]
    E, I2, _ = w13q.shape
    I = I2 // 2
    _need(xq, "xq", _U8, (T, H))
    _need(xs, "xs", _U8, (T, H // 32))
    _need(topk_ids, "topk_ids", (torch.int32,), (T, topk))
    _need(topk_w, "topk_w", _F32, (T, topk))
    _need(w13q, "w13q", _U8, (E, 2 * I, H))
    _need(w13s, "w13s", _U8, (E, 2 * I, H // 32))
    _need(w2q, "w2q", _U8, (E, H, I))
    _need(w2s, "w2s", _U8, (E, H, I // 32))
    _need(out, "out", (torch.bfloat16,), (T, H))
    if dbg_h is not None:
        _need(dbg_h, "dbg_h", _U8, numel=T * topk * (I + I // 32))
    need = mgemm_workspace_bytes(OP_MOE, T=T, H=H, I=I, E=E, topk=topk)
    if ws is None:
        ws = workspace(need, "moe", stream)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("moe: workspace too small")
    if dbg_gu is not None:
        _need(dbg_gu, "dbg_gu", _F32, numel=T * topk * 2 * I)
        _check("mgemm_moe_mxfp8_glu_debug", load().mgemm_moe_mxfp8_glu_debug(
            xq.data_ptr(), xs.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), T, H, I, E,
            topk, w13q.data_ptr(), w13s.data_ptr(), w2q.data_ptr(), w2s.data_ptr(),
            out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
            dbg_h.data_ptr() if dbg_h is not None else None, dbg_gu.data_ptr(), _stream(stream)))
        return out
    _check("mgemm_moe_mxfp8_glu", load().mgemm_moe_mxfp8_glu(
        xq.data_ptr(), xs.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), T, H, I, E, topk,
        w13q.data_ptr(), w13s.data_ptr(), w2q.data_ptr(), w2s.data_ptr(), out.data_ptr(),
        ws.data_ptr(), ws.numel() * ws.element_size(),
        dbg_h.data_ptr() if dbg_h is not None else None, _stream(stream)))
    return out


def mgemm_moe_mxfp8_glu_logits(xq, xs, logits, topk, w13q, w13s, w2q, w2s, out,
                               topk_ids=None, topk_w=None, ws: Optional[torch.Tensor] = None,
                               dbg_h: Optional[torch.Tensor] = None, stream=None):
    """The MXFP8 MoE routed from FP32 router logits [T,E] in the same call
    (softmax, top-k, expert counts in the route-prep launch).  Returns
    (out, topk_ids, topk_w): the routing the call took, [T,topk]."""
    T, H = xq.shape
    E, I2, _ = w13q.shape
    I = I2 // 2
    _need(xq, "xq", _U8, (T, H))
    _need(xs, "xs", _U8, (T, H // 32))
    _need(logits, "logits", _F32, (T, E))
    _need(w13q, "w13q", _U8, (E, 2 * I, H))
    _need(w13s, "w13s", _U8, (E, 2 * I, H // 32))
    _need(w2q, "w2q", _U8, (E, H, I))
    _need(w2s, "w2s", _U8, (E, H, I // 32))
    _need(out, "out", (torch.bfloat16,), (T, H))
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=xq.device)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=xq.device)
    _need(topk_ids, "topk_ids", (torch.int32,), (T, topk))
    _need(topk_w, "topk_w", _F32, (T, topk))
    if dbg_h is not None:
        _need(dbg_h, "dbg_h", _U8, numel=T * topk * (I + I // 32))
    need = mgemm_workspace_bytes(OP_MOE, T=T, H=H, I=I, E=E, topk=topk)
    if ws is None:
        ws = workspace(need, "moe", stream)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("moe: workspace too small")
    _check("mgemm_moe_mxfp8_glu_logits", load().mgemm_moe_mxfp8_glu_logits(
        xq.data_ptr(), xs.data_ptr(), logits.data_ptr(), T, H, I, E, topk, w13q.data_ptr(),
        w13s.data_ptr(), w2q.data_ptr(), w2s.data_ptr(), out.data_ptr(), topk_ids.data_ptr(),
        topk_w.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
        dbg_h.data_ptr() if dbg_h is not None else None, _stream(stream)))
    return out, topk_ids, topk_w


def mgemm_moe_nvfp4_glu(xq, xs, Sx, topk_ids, topk_w, w13q, w13s, Sw13, w2q, w2s, Sw2, Sh, out,
                        ws: Optional[torch.Tensor] = None, dbg_h: Optional[torch.Tensor] = None,
                        stream=None):
    """NVFP4 grouped MoE GLU; Sx, Sh: FP32 [1], Sw13, Sw2: FP32 [E] (device)."""
    T, H2 = xq.shape
    H = 2 * H2
    topk = topk_ids.shape[1]
    E, I2, _ = w13q.shape
    I = I2 // 2
    _need(xq, "xq", _U8, (T, H // 2))
    _need(xs, "xs", _U8, (T, H // 16))
    _need(Sx, "Sx", _F32, numel=1)
    _need(topk_ids, "topk_ids", (torch.int32,), (T, topk))
    _need(topk_w, "topk_w", _F32, (T, topk))
    _need(w13q, "w13q", _U8, (E, 2 * I, H // 2))
    _need(w13s, "w13s", _U8, (E, 2 * I, H // 16))
    _need(Sw13, "Sw13", _F32, numel=E)
    _need(w2q, "w2q", _U8, (E, H, I // 2))
    _need(w2s, "w2s", _U8, (E, H, I // 16))
    _need(Sw2, "Sw2", _F32, numel=E)
    _need(Sh, "Sh", _F32, numel=1)
    _need(out, "out", (torch.bfloat16,), (T, H))
    if dbg_h is not None:
        _need(dbg_h, "dbg_h", _U8, numel=T * topk * (I // 2 + I // 16))
    need = mgemm_workspace_bytes(OP_MOE_NVFP4, T=T, H=H, I=I, E=E, topk=topk)
    if ws is None:
        ws = workspace(need, "moe_nvfp4", stream)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("moe_nvfp4: workspace too small")
    _check("mgemm_moe_nvfp4_glu", load().mgemm_moe_nvfp4_glu(
        xq.data_ptr(), xs.data_ptr(), Sx.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(),
        T, H, I, E, topk, w13q.data_ptr(), w13s.data_ptr(), Sw13.data_ptr(), w2q.data_ptr(),
        w2s.data_ptr(), Sw2.data_ptr(), Sh.data_ptr(), out.data_ptr(), ws.data_ptr(),
        ws.numel() * ws.element_size(), dbg_h.data_ptr() if dbg_h is not None else None,
        _stream(stream)))
    return out


def mgemm_moe_route_topk(logits, topk, topk_ids=None, topk_w=None, stream=None):
    """(ids int32 [T,topk], weights FP32 [T,topk]) from FP32 router logits [T,E]."""
    T, E = logits.shape
    _need(logits, "logits", _F32, (T, E))
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    _need(topk_ids, "topk_ids", (torch.int32,), (T, topk))
    _need(topk_w, "topk_w", _F32, (T, topk))
    _check("mgemm_moe_route_topk", load().mgemm_moe_route_topk(
        logits.data_ptr(), T, E, topk, topk_ids.data_ptr(), topk_w.data_ptr(), _stream(stream)))
    return topk_ids, topk_w


def mgemm_bf16_dgrad(dY, W, dX=None, out_f32=False, ws: Optional[torch.Tensor] = None, stream=None):
    """dX[M,K] = dY[M,N] . W[N,K] (BF16 in, BF16 or FP32 out)."""
    M, N = dY.shape
    _, K = W.shape
    _need(dY, "dY", (torch.bfloat16,), (M, N))
    _need(W, "W", (torch.bfloat16,), (N, K))
    if dX is None:
        dX = torch.empty((M, K), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dY.device)
    _need(dX, "dX", (torch.float32 if out_f32 else torch.bfloat16,), (M, K))
    need = mgemm_workspace_bytes(OP_BF16_DGRAD, M, N, K)
    if ws is None:
        ws = workspace(need, "bf16_dgrad", stream)
    _check("mgemm_bf16_dgrad", load().mgemm_bf16_dgrad(
        dY.data_ptr(), W.data_ptr(), dX.data_ptr(), M, N, K, int(out_f32),
        ws.data_ptr() if ws is not None else None,
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))
    return dX


def mgemm_bf16_wgrad(dY, X, dW=None, out_f32=False, ws: Optional[torch.Tensor] = None, stream=None):
    """dW[N,K] = dY[M,N]^T . X[M,K] (BF16 in, BF16 or FP32 out)."""
    M, N = dY.shape
    _, K = X.shape
    _need(dY, "dY", (torch.bfloat16,), (M, N))
    _need(X, "X", (torch.bfloat16,), (M, K))
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32 if out_f32 else torch.bfloat16, device=dY.device)
    _need(dW, "dW", (torch.float32 if out_f32 else torch.bfloat16,), (N, K))
    need = mgemm_workspace_bytes(OP_BF16_WGRAD, M, N, K)
    if ws is None:
        ws = workspace(need, "bf16_wgrad", stream)
    _check("mgemm_bf16_wgrad", load().mgemm_bf16_wgrad(
        dY.data_ptr(), X.data_ptr(), dW.data_ptr(), M, N, K, int(out_f32),
        ws.data_ptr() if ws is not None else None,
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))
    return dW
