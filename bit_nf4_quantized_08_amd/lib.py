"""Thin Python binding of ``libqlora_nf4.so`` (argument marshalling only).

Every function here checks dtypes/devices/shapes of torch tensors, hands raw
device pointers, sizes and torch's current HIP stream to the C ABI declared in
``include/qlora_nf4.h``, and raises on a non-zero status.  All arithmetic runs
in the library's HIP kernels; there is no CPU or PyTorch fallback.

Names follow the C ABI: ``nf4_quantize``, ``nf4_double_quant``, ``nf4_dequant``,
``qlora_linear_fwd``, ``qlora_linear_bwd``, plus ``qn_codebook``.
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlora_nf4.so")

QN_OK = 0
QN_F32, QN_BF16 = 0, 1
QN_OP_FWD, QN_OP_BWD = 0, 1
QN_BLOCK, QN_GROUP, QN_MAX_RANK = 64, 256, 64

_lib = None


class QNError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


class NF4WeightStruct(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("scale2", ctypes.c_void_p),
        ("N", ctypes.c_int64),
        ("K", ctypes.c_int64),
    ]


def load():
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bit_nf4_quantized_08_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sig = {
        "qn_codebook": (i32, [ctypes.POINTER(ctypes.c_float)]),
        "nf4_quantize": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "nf4_double_quant": (i32, [vp, i64, vp, vp, vp]),
        "nf4_dequant": (i32, [ctypes.POINTER(NF4WeightStruct), vp, i32, vp]),
        "qlora_workspace_size": (ctypes.c_size_t, [i32, i64, i64, i64, i64]),
        "qlora_linear_fwd": (i32, [vp, i64, ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, vp, vp,
                                   ctypes.c_size_t, vp]),
        "qlora_linear_bwd": (i32, [vp, vp, i64, ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, vp, vp,
                                   vp, ctypes.c_size_t, vp]),
        "qn_status_string": (ctypes.c_char_p, [i32]),
        "qn_trace_enable": (i32, [i32]),
        "qn_trace_read": (i32, [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float), i32]),
        "qn_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return ["qn_codebook", "nf4_quantize", "nf4_double_quant", "nf4_dequant", "qlora_workspace_size",
            "qlora_linear_fwd", "qlora_linear_bwd", "qn_status_string", "qn_version", "qn_trace_enable",
            "qn_trace_read"]


def status_string(status):
    return load().qn_status_string(int(status)).decode()


def _check(fn, status):
    if status != QN_OK:
        raise QNError(fn, status)


def qn_codebook():
    """The library's NF4 table (host call, no device work): numpy float32[16]."""
    out = (ctypes.c_float * 16)()
    _check("qn_codebook", load().qn_codebook(out))
    return np.frombuffer(out, dtype=np.float32).copy()


# ------------------------------------------------------------------ torch glue
def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype=None, ndim=None, device_cuda=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device_cuda and t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got {t.dim()}-D")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclass
class NF4Weight:
    """A frozen weight W[N, K] in NF4 form (device tensors)."""
    codes: "object"                 # uint8 [ceil(N*K/2)]
    absmax: Optional[object]        # fp32 [nb] (kept after double quantisation too)
    absmax_q: Optional[object]      # uint8 [nb] or None
    scale2: Optional[object]        # fp32 [ceil(nb/256)] or None
    N: int
    K: int

    def struct(self, use_double_quant=True):
        dq = use_double_quant and self.absmax_q is not None
        return NF4WeightStruct(
            self.codes.data_ptr(),
            self.absmax.data_ptr() if (self.absmax is not None and not dq) else 0,
            self.absmax_q.data_ptr() if dq else 0,
            self.scale2.data_ptr() if dq else 0,
            self.N, self.K)


def nf4_quantize(W, codes=None, absmax=None):
    """Blockwise NF4 quantisation of a 2-D fp32 or bf16 device tensor."""
    torch = _torch()
    _need(W, "W", ndim=2)
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("W must be float32 or bfloat16")
    N, K = W.shape
    n = N * K
    if codes is None:
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=W.device)
    if absmax is None:
        absmax = torch.empty((n + 63) // 64, dtype=torch.float32, device=W.device)
    dt = QN_BF16 if W.dtype == torch.bfloat16 else QN_F32
    _check("nf4_quantize", load().nf4_quantize(_ptr(W), dt, N, K, _ptr(codes), _ptr(absmax), _stream()))
    return codes, absmax


def nf4_double_quant(absmax, absmax_q=None, scale2=None):
    torch = _torch()
    _need(absmax, "absmax", dtype=torch.float32, ndim=1)
    nb = absmax.numel()
    if absmax_q is None:
        absmax_q = torch.empty(nb, dtype=torch.uint8, device=absmax.device)
    if scale2 is None:
        scale2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=absmax.device)
    _check("nf4_double_quant", load().nf4_double_quant(_ptr(absmax), nb, _ptr(absmax_q), _ptr(scale2), _stream()))
    return absmax_q, scale2


def quantize_weight(W, double_quant=True):
    """W (2-D device tensor) -> NF4Weight, optionally double-quantised."""
    codes, absmax = nf4_quantize(W)
    aq = s2 = None
    if double_quant:
        aq, s2 = nf4_double_quant(absmax)
    return NF4Weight(codes, absmax, aq, s2, int(W.shape[0]), int(W.shape[1]))


def nf4_dequant(w: NF4Weight, out_dtype="bf16", use_double_quant=True, out=None):
    torch = _torch()
    dt = {"bf16": (QN_BF16, torch.bfloat16), "f32": (QN_F32, torch.float32)}[out_dtype]
    if out is None:
        out = torch.empty((w.N, w.K), dtype=dt[1], device=w.codes.device)
    st = w.struct(use_double_quant)
    _check("nf4_dequant", load().nf4_dequant(ctypes.byref(st), _ptr(out), dt[0], _stream()))
    return out


def workspace_size(op, M, N, K, r):
    return int(load().qlora_workspace_size(op, M, N, K, r))


def workspace(op, M, N, K, r, device="cuda"):
    torch = _torch()
    nbytes = workspace_size(op, M, N, K, r)
    if nbytes == 0:
        raise QNError("qlora_workspace_size", 2)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_linear_fwd(X, w: NF4Weight, A, B, alpha, want_H=False, use_double_quant=True, Y=None, ws=None):
    """Y = X bf16(dequant(W))^T + (alpha/r) (X A^T) B^T; returns Y (and H)."""
    torch = _torch()
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = X.shape
    r = A.shape[0]
    if K != w.K or A.shape[1] != w.K or B.shape != (w.N, r):
        raise ValueError("shape mismatch between X, W, A, B")
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=X.device)
    H = torch.empty((M, r), dtype=torch.float32, device=X.device) if want_H else None
    if ws is None:
        ws = workspace(QN_OP_FWD, M, w.N, w.K, r, X.device)
    st = w.struct(use_double_quant)
    _check("qlora_linear_fwd", load().qlora_linear_fwd(
        _ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(H),
        _ptr(ws), ws.numel(), _stream()))
    return (Y, H) if want_H else Y


def qlora_linear_bwd(dY, X, w: NF4Weight, A, B, alpha, want_dX=True, use_double_quant=True, out=None, ws=None):
    """Returns (dX or None, dA, dB) for the upstream gradient dY."""
    torch = _torch()
    _need(dY, "dY", torch.bfloat16, 2)
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = X.shape
    r = A.shape[0]
    if dY.shape != (M, w.N) or K != w.K or A.shape[1] != w.K or B.shape != (w.N, r):
        raise ValueError("shape mismatch between dY, X, W, A, B")
    if out is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device) if want_dX else None
        dA = torch.empty((r, K), dtype=torch.bfloat16, device=X.device)
        dB = torch.empty((w.N, r), dtype=torch.bfloat16, device=X.device)
    else:
        dX, dA, dB = out
    if ws is None:
        ws = workspace(QN_OP_BWD, M, w.N, w.K, r, X.device)
    st = w.struct(use_double_quant)
    _check("qlora_linear_bwd", load().qlora_linear_bwd(
        _ptr(dY), _ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(dX), _ptr(dA),
        _ptr(dB), _ptr(ws), ws.numel(), _stream()))
    return dX, dA, dB


TRACE_KINDS = {1: "quantize", 2: "double_quant", 3: "dequant", 4: "gemv", 5: "gemm_fwd", 6: "gemm_dx",
               7: "gemm_db", 8: "gemm_da", 9: "lowrank"}


def trace_enable(on=True):
    _check("qn_trace_enable", load().qn_trace_enable(1 if on else 0))


def trace_read(cap=1 << 16):
    """Wait for the logged kernels; returns a list of (kind name, milliseconds)."""
    kinds = (ctypes.c_int * cap)()
    ms = (ctypes.c_float * cap)()
    n = load().qn_trace_read(kinds, ms, cap)
    if n < 0:
        raise QNError("qn_trace_read", -n)
    return [(TRACE_KINDS.get(kinds[i], str(kinds[i])), float(ms[i])) for i in range(n)]


def raw():
    """The ctypes library object (for callers passing raw pointers)."""
    return load()
