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
# QN_LIBRARY names another build of the same library (the host-sanitizer build
# that the ABI tests load in a child process); by default the in-tree one.
LIB_PATH = os.environ.get("QN_LIBRARY") or os.path.join(_PKG, "libqlora_nf4.so")

QN_OK = 0
QN_F32, QN_BF16 = 0, 1
QN_NF4, QN_FP4 = 0, 1
QUANT_TYPES = {"nf4": QN_NF4, "fp4": QN_FP4}
QN_OP_FWD, QN_OP_BWD = 0, 1
QN_ERR_SCRATCH = 8
QN_ERR_MEMORY = 9
QN_NOALLOC_SCRATCH_BYTES = 16 << 20
QN_BLOCK, QN_GROUP, QN_MAX_RANK, QN_MAX_GROUP = 64, 256, 64, 8
QN_ADAMW_MULTI = 32

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
        ("quant_type", ctypes.c_int32),
    ]


class FwdProblemStruct(ctypes.Structure):
    _fields_ = [
        ("X", ctypes.c_void_p),
        ("M", ctypes.c_int64),
        ("W", NF4WeightStruct),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("r", ctypes.c_int64),
        ("alpha", ctypes.c_float),
        ("Y", ctypes.c_void_p),
        ("H_out", ctypes.c_void_p),
    ]


class AdamWConfigStruct(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int64),
    ]


class AdamWTensorStruct(ctypes.Structure):
    """qn_adamw_tensor: one tensor of a multi-tensor step."""
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("m_q", ctypes.c_void_p), ("m_step", ctypes.c_void_p), ("u_q", ctypes.c_void_p),
                ("u_step", ctypes.c_void_p)]


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
        "qn_table": (i32, [i32, ctypes.POINTER(ctypes.c_float)]),
        "qn_quantize_4bit": (i32, [vp, i32, i64, i64, i32, vp, vp, vp, vp, vp]),
        "nf4_quantize": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "nf4_double_quant": (i32, [vp, i64, vp, vp, vp]),
        "nf4_dequant": (i32, [ctypes.POINTER(NF4WeightStruct), vp, i32, vp]),
        "qn_adamw8_step": (i32, [vp, vp, i64, vp, vp, vp, vp, ctypes.POINTER(AdamWConfigStruct), vp]),
        "qn_adamw8_step_multi": (i32, [i32, ctypes.POINTER(AdamWTensorStruct), ctypes.POINTER(AdamWConfigStruct), vp]),
        "qlora_merge": (i32, [ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, i32, vp]),
        "qlora_workspace_size": (ctypes.c_size_t, [i32, i64, i64, i64, i64]),
        "qlora_linear_fwd": (i32, [vp, i64, ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, vp, vp,
                                   ctypes.c_size_t, vp]),
        "qlora_workspace_size_grouped": (ctypes.c_size_t, [i32, ctypes.POINTER(FwdProblemStruct)]),
        "qlora_linear_fwd_grouped": (i32, [i32, ctypes.POINTER(FwdProblemStruct), vp, ctypes.c_size_t, vp]),
        "qlora_linear_fwd_noalloc": (i32, [vp, i64, ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, vp, vp]),
        "qlora_linear_bwd": (i32, [vp, vp, vp, i64, ctypes.POINTER(NF4WeightStruct), vp, vp, i64, f32, vp, vp,
                                   vp, vp, ctypes.c_size_t, vp]),
        "qn_status_string": (ctypes.c_char_p, [i32]),
        "qn_trace_enable": (i32, [i32]),
        "qn_set_gemm_variant": (i32, [i32]),
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
    return ["qn_codebook", "qn_table", "qn_quantize_4bit", "nf4_quantize", "nf4_double_quant", "nf4_dequant", "qlora_merge", "qn_adamw8_step", "qn_adamw8_step_multi",
            "qlora_workspace_size",
            "qlora_linear_fwd", "qlora_linear_fwd_noalloc", "qlora_workspace_size_grouped",
            "qlora_linear_fwd_grouped", "qlora_linear_bwd", "qn_status_string", "qn_version", "qn_set_gemm_variant", "qn_trace_enable",
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


def qn_table(quant_type="nf4"):
    """The library's table of a 4-bit type ("nf4" or "fp4"), by code: numpy float32[16]."""
    out = (ctypes.c_float * 16)()
    _check("qn_table", load().qn_table(QUANT_TYPES[quant_type], out))
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
    quant_type: int = QN_NF4        # QN_NF4 or QN_FP4: the table the codes index

    def struct(self, use_double_quant=True):
        dq = use_double_quant and self.absmax_q is not None
        return NF4WeightStruct(
            self.codes.data_ptr(),
            self.absmax.data_ptr() if (self.absmax is not None and not dq) else 0,
            self.absmax_q.data_ptr() if dq else 0,
            self.scale2.data_ptr() if dq else 0,
            self.N, self.K, self.quant_type)


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


def quantize_4bit(W, quant_type="nf4", codes=None, absmax=None, absmax_q=None, scale2=None, double_quant=True):
    """qn_quantize_4bit: blockwise 4-bit quantisation of a 2-D fp32 or bf16 device
    tensor, with the block scales double-quantised in the same launch when
    ``double_quant``.  Returns an NF4Weight (absmax kept either way)."""
    torch = _torch()
    _need(W, "W", ndim=2)
    if W.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("W must be float32 or bfloat16")
    N, K = W.shape
    n = N * K
    nb = (n + 63) // 64
    if codes is None:
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=W.device)
    if absmax is None:
        absmax = torch.empty(nb, dtype=torch.float32, device=W.device)
    if double_quant:
        if absmax_q is None:
            absmax_q = torch.empty(nb, dtype=torch.uint8, device=W.device)
        if scale2 is None:
            scale2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=W.device)
    else:
        absmax_q = scale2 = None
    dt = QN_BF16 if W.dtype == torch.bfloat16 else QN_F32
    qt = QUANT_TYPES[quant_type]
    _check("qn_quantize_4bit", load().qn_quantize_4bit(_ptr(W), dt, N, K, qt, _ptr(codes), _ptr(absmax),
                                                       _ptr(absmax_q), _ptr(scale2), _stream()))
    return NF4Weight(codes, absmax, absmax_q, scale2, int(N), int(K), qt)


def quantize_weight(W, double_quant=True, quant_type="nf4", fused=True):
    """W (2-D device tensor) -> NF4Weight, optionally double-quantised: by default
    in one launch (qn_quantize_4bit); ``fused=False`` (NF4 only) runs
    nf4_quantize and then nf4_double_quant."""
    if fused or quant_type != "nf4":
        return quantize_4bit(W, quant_type, double_quant=double_quant)
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


def qlora_merge(w: NF4Weight, A, B, alpha, out_dtype="bf16", use_double_quant=True, out=None):
    """The adapter merged into the dequantised base: [N, K] bf16 (or fp32)."""
    torch = _torch()
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    r = A.shape[0]
    if A.shape[1] != w.K or B.shape != (w.N, r):
        raise ValueError("A must be [r, K] and B [N, r]")
    dt = {"bf16": (QN_BF16, torch.bfloat16), "f32": (QN_F32, torch.float32)}[out_dtype]
    if out is None:
        out = torch.empty((w.N, w.K), dtype=dt[1], device=w.codes.device)
    st = w.struct(use_double_quant)
    _check("qlora_merge", load().qlora_merge(ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(out), dt[0],
                                             _stream()))
    return out


class AdamW8State:
    """8-bit block-wise AdamW state of one bf16 tensor (zeros: before the first step).

    host=True places the state in pinned host memory mapped for the device
    (the "paged" placement: none of its bytes occupy device memory, and the
    step reads and writes it across the host link)."""

    def __init__(self, n, device="cuda", host=False):
        torch = _torch()
        nb = (n + 63) // 64
        self.n = n
        self.host = bool(host)
        kw = dict(device="cpu", pin_memory=True) if self.host else dict(device=device)
        self.m_q = torch.zeros(n, dtype=torch.int8, **kw)
        self.m_step = torch.zeros(nb, dtype=torch.float32, **kw)
        self.u_q = torch.zeros(n, dtype=torch.uint8, **kw)
        self.u_step = torch.zeros(nb, dtype=torch.float32, **kw)
        self.step = 0


def adamw8_step(param, grad, state: AdamW8State, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                step=None):
    """One qn_adamw8_step on a bf16 tensor in place; advances state.step
    unless an explicit step number is given."""
    torch = _torch()
    _need(param, "param", torch.bfloat16)
    _need(grad, "grad", torch.bfloat16)
    if param.numel() != state.n or grad.numel() != state.n:
        raise ValueError("param, grad and state sizes differ")
    if step is None:
        state.step += 1
        step = state.step
    cfg = AdamWConfigStruct(lr, beta1, beta2, eps, weight_decay, int(step))
    _check("qn_adamw8_step", load().qn_adamw8_step(
        _ptr(param), _ptr(grad), state.n, _ptr(state.m_q), _ptr(state.m_step), _ptr(state.u_q), _ptr(state.u_step),
        ctypes.byref(cfg), _stream()))
    return param


def adamw8_step_multi(params, grads, states, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                      step=None):
    """One qn_adamw8_step_multi over several bf16 tensors in place (one launch
    per QN_ADAMW_MULTI tensors); all states advance to the same step unless an
    explicit step number is given."""
    torch = _torch()
    if not (len(params) == len(grads) == len(states)) or not params:
        raise ValueError("params, grads and states must be non-empty lists of one length")
    arr = (AdamWTensorStruct * len(params))()
    for i, (p, g, st) in enumerate(zip(params, grads, states)):
        _need(p, "param", torch.bfloat16)
        _need(g, "grad", torch.bfloat16)
        if p.numel() != st.n or g.numel() != st.n:
            raise ValueError("param, grad and state sizes differ")
        arr[i] = AdamWTensorStruct(_ptr(p), _ptr(g), st.n, _ptr(st.m_q), _ptr(st.m_step), _ptr(st.u_q),
                                   _ptr(st.u_step))
    if step is None:
        step = states[0].step + 1
    for st in states:
        st.step = int(step)
    cfg = AdamWConfigStruct(lr, beta1, beta2, eps, weight_decay, int(step))
    _check("qn_adamw8_step_multi", load().qn_adamw8_step_multi(len(params), arr, ctypes.byref(cfg), _stream()))
    return params


def workspace_size(op, M, N, K, r):
    return int(load().qlora_workspace_size(op, M, N, K, r))


def workspace(op, M, N, K, r, device="cuda"):
    torch = _torch()
    nbytes = workspace_size(op, M, N, K, r)
    if nbytes == 0:
        raise QNError("qlora_workspace_size", 2)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def qlora_linear_fwd(X, w: NF4Weight, A, B, alpha, want_H=False, use_double_quant=True, Y=None, ws=None, H=None):
    """Y = X bf16(dequant(W))^T + (alpha/r) (X A^T) B^T; returns Y (and H).

    ``H`` (optional, fp32 [M, r]) receives X A^T; passing it implies want_H."""
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
    _need(Y, "Y", torch.bfloat16, 2)
    if Y.shape != (M, w.N):
        raise ValueError("Y must be [M, N]")
    if H is not None:
        _need(H, "H", torch.float32, 2)
        if H.shape != (M, r):
            raise ValueError("H must be [M, r]")
        want_H = True
    elif want_H:
        H = torch.empty((M, r), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(QN_OP_FWD, M, w.N, w.K, r, X.device)
    st = w.struct(use_double_quant)
    _check("qlora_linear_fwd", load().qlora_linear_fwd(
        _ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(H),
        _ptr(ws), ws.numel(), _stream()))
    return (Y, H) if want_H else Y


class FwdGroup:
    """A fixed set of independent forwards for qlora_linear_fwd_grouped.

    ``problems`` is a list of (X, w, A, B, alpha, Y, H) with H optional (None);
    the descriptor array and the workspace are built once, so that run() only
    enqueues (and can be captured into a HIP graph)."""

    def __init__(self, problems, use_double_quant=True, ws=None):
        torch = _torch()
        n = len(problems)
        if not 1 <= n <= QN_MAX_GROUP:
            raise ValueError(f"1 to {QN_MAX_GROUP} problems per group")
        self._keep = problems
        arr = (FwdProblemStruct * n)()
        for i, (X, w, A, B, alpha, Y, H) in enumerate(problems):
            _need(X, "X", torch.bfloat16, 2)
            _need(A, "A", torch.bfloat16, 2)
            _need(B, "B", torch.bfloat16, 2)
            _need(Y, "Y", torch.bfloat16, 2)
            M, K = X.shape
            r = A.shape[0]
            if K != w.K or A.shape[1] != w.K or B.shape != (w.N, r) or Y.shape != (M, w.N):
                raise ValueError(f"problem {i}: shape mismatch between X, W, A, B, Y")
            if H is not None:
                _need(H, "H", torch.float32, 2)
                if H.shape != (M, r):
                    raise ValueError(f"problem {i}: H must be [M, r]")
            arr[i] = FwdProblemStruct(X.data_ptr(), M, w.struct(use_double_quant), A.data_ptr(), B.data_ptr(), r,
                                      float(alpha), Y.data_ptr(), H.data_ptr() if H is not None else 0)
        self._arr, self._n = arr, n
        nbytes = int(load().qlora_workspace_size_grouped(n, arr))
        if nbytes == 0:
            raise QNError("qlora_workspace_size_grouped", 2)
        self.ws = ws if ws is not None else torch.empty(nbytes, dtype=torch.uint8, device=problems[0][0].device)

    def run(self):
        _check("qlora_linear_fwd_grouped", load().qlora_linear_fwd_grouped(
            self._n, self._arr, _ptr(self.ws), self.ws.numel(), _stream()))


def qlora_linear_fwd_grouped(problems, use_double_quant=True):
    """Run independent forwards [(X, w, A, B, alpha, Y, H or None), ...] in one call."""
    FwdGroup(problems, use_double_quant).run()


def qlora_linear_fwd_noalloc(X, w: NF4Weight, A, B, alpha, Y, H=None, use_double_quant=True):
    """qlora_linear_fwd without a workspace: the library's static scratch array
    is the workspace.  Y (and H) are caller-provided; nothing is allocated."""
    torch = _torch()
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    _need(Y, "Y", torch.bfloat16, 2)
    M, K = X.shape
    r = A.shape[0]
    if K != w.K or A.shape[1] != w.K or B.shape != (w.N, r) or Y.shape != (M, w.N):
        raise ValueError("shape mismatch between X, W, A, B, Y")
    if H is not None:
        _need(H, "H", torch.float32, 2)
        if H.shape != (M, r):
            raise ValueError("H must be [M, r]")
    st = w.struct(use_double_quant)
    _check("qlora_linear_fwd_noalloc", load().qlora_linear_fwd_noalloc(
        _ptr(X), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(Y), _ptr(H), _stream()))
    return Y


def qlora_linear_bwd(dY, X, w: NF4Weight, A, B, alpha, want_dX=True, use_double_quant=True, out=None, ws=None,
                     H=None):
    """Returns (dX or None, dA, dB) for the upstream gradient dY.

    ``H`` (optional, fp32 [M, r]) is X A^T as the forward returned it with
    ``want_H=True``; given, the call does not recompute it from X."""
    torch = _torch()
    _need(dY, "dY", torch.bfloat16, 2)
    _need(X, "X", torch.bfloat16, 2)
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = X.shape
    r = A.shape[0]
    if dY.shape != (M, w.N) or K != w.K or A.shape[1] != w.K or B.shape != (w.N, r):
        raise ValueError("shape mismatch between dY, X, W, A, B")
    if H is not None:
        _need(H, "H", torch.float32, 2)
        if H.shape != (M, r):
            raise ValueError("H must be [M, r]")
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
        _ptr(dY), _ptr(X), _ptr(H), M, ctypes.byref(st), _ptr(A), _ptr(B), r, float(alpha), _ptr(dX), _ptr(dA),
        _ptr(dB), _ptr(ws), ws.numel(), _stream()))
    return dX, dA, dB


TRACE_KINDS = {1: "quantize", 2: "double_quant", 3: "dequant", 4: "gemv", 5: "gemm_fwd", 6: "gemm_dx",
               7: "gemm_db", 8: "gemm_da", 9: "lowrank", 10: "merge", 11: "adamw8"}


def set_gemm_variant(variant):
    """Forward dequant-GEMM tiling for later calls: 0 automatic, 1 256x128, 2 256x256."""
    _check("qn_set_gemm_variant", load().qn_set_gemm_variant(int(variant)))


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
