"""CPU-only checks of the C ABI: the library loads, exports what the header
declares, derives the same NF4 table as the oracle (two independent
derivations), and rejects bad arguments on the host before launching anything.
No call here reaches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from bit_nf4_quantized_08_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lib.LIB_PATH), reason="library not built")

FAKE = 0x10000  # 16-byte aligned fake device address: never dereferenced by a rejected call
MISALIGNED = FAKE + 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_symbols_are_exported():
    L = lib.load()
    decl = declared_functions()
    assert set(decl) >= {"nf4_quantize", "nf4_double_quant", "nf4_dequant", "qlora_linear_fwd",
                         "qlora_linear_bwd", "qn_codebook"}
    for name in decl:
        assert hasattr(L, name), name
    assert set(decl) == set(lib.exported_symbols())


def test_library_table_equals_oracle_bits():
    """The library derives the table by Newton's method on erfc; the oracle by the
    standard library's inverse normal CDF.  The fp32 bits must agree."""
    np.testing.assert_array_equal(lib.qn_codebook().view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_status_strings():
    assert lib.status_string(0) == "ok"
    assert "null" in lib.status_string(1)
    assert lib.status_string(99) == "unknown status"
    assert "pinned host memory" in lib.status_string(lib.QN_ERR_MEMORY)


def _w(N=64, K=64, codes=FAKE, absmax=FAKE, absmax_q=0, scale2=0, quant_type=0):
    return lib.NF4WeightStruct(codes, absmax, absmax_q, scale2, N, K, quant_type)


def test_quantize_rejects_bad_arguments():
    L = lib.load()
    vp = ctypes.c_void_p
    assert L.nf4_quantize(vp(0), 0, 4, 4, vp(FAKE), vp(FAKE), vp(0)) == 1
    assert L.nf4_quantize(vp(FAKE), 7, 4, 4, vp(FAKE), vp(FAKE), vp(0)) == 3
    assert L.nf4_quantize(vp(FAKE), 0, 0, 4, vp(FAKE), vp(FAKE), vp(0)) == 2
    assert L.nf4_quantize(vp(FAKE), 0, -1, 4, vp(FAKE), vp(FAKE), vp(0)) == 2
    assert L.nf4_quantize(vp(MISALIGNED), 0, 4, 4, vp(FAKE), vp(FAKE), vp(0)) == 4
    assert L.nf4_quantize(vp(FAKE), 1, 1 << 30, 1 << 30, vp(FAKE), vp(FAKE), vp(0)) == 2


def test_double_quant_and_dequant_reject_bad_arguments():
    L = lib.load()
    vp = ctypes.c_void_p
    assert L.nf4_double_quant(vp(0), 10, vp(FAKE), vp(FAKE), vp(0)) == 1
    assert L.nf4_double_quant(vp(FAKE), 0, vp(FAKE), vp(FAKE), vp(0)) == 2
    assert L.nf4_dequant(None, vp(FAKE), 0, vp(0)) == 1
    w = _w(codes=0)
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 1
    w = _w(absmax=0)
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 1
    w = _w(absmax=0, absmax_q=FAKE, scale2=0)          # double quant needs scale2
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 1
    w = _w()
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 5, vp(0)) == 3
    assert L.nf4_dequant(ctypes.byref(w), vp(MISALIGNED), 0, vp(0)) == 4
    w = _w(codes=MISALIGNED)
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 4
    w = _w(absmax=0, absmax_q=FAKE + 1, scale2=FAKE)   # 8-bit scales are read as aligned words
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 4


def test_workspace_size_rules():
    assert lib.workspace_size(lib.QN_OP_FWD, 2048, 4096, 4096, 16) > 0
    assert lib.workspace_size(lib.QN_OP_FWD, 1, 4096, 4096, 16) > 0
    assert lib.workspace_size(lib.QN_OP_BWD, 4, 256, 512, 8) > 0
    assert lib.workspace_size(lib.QN_OP_FWD, 0, 4096, 4096, 16) == 0
    assert lib.workspace_size(lib.QN_OP_FWD, 8, 4096, 4000, 16) == 0      # K % 64
    assert lib.workspace_size(lib.QN_OP_FWD, 8, 4000, 4096, 16) == 0      # N % 64
    assert lib.workspace_size(lib.QN_OP_FWD, 8, 4096, 4096, 65) == 0      # r > 64
    assert lib.workspace_size(7, 8, 4096, 4096, 16) == 0


def test_linear_rejects_bad_arguments():
    L = lib.load()
    vp = ctypes.c_void_p
    w = _w(N=256, K=512)
    big = 1 << 40
    args = lambda M=4, r=8, alpha=16.0, ws=FAKE, wsb=big, X=FAKE: (
        vp(X), M, ctypes.byref(w), vp(FAKE), vp(FAKE), r, alpha, vp(FAKE), vp(0), vp(ws), wsb, vp(0))
    assert L.qlora_linear_fwd(*args(X=0)) == 1
    assert L.qlora_linear_fwd(*args(M=0)) == 2
    assert L.qlora_linear_fwd(*args(r=0)) == 2
    assert L.qlora_linear_fwd(*args(r=65)) == 2
    assert L.qlora_linear_fwd(*args(alpha=float("nan"))) == 7
    assert L.qlora_linear_fwd(*args(ws=0)) == 5
    assert L.qlora_linear_fwd(*args(wsb=16)) == 5
    assert L.qlora_linear_fwd(*args(X=MISALIGNED)) == 4
    w2 = _w(N=256, K=500)
    assert L.qlora_linear_fwd(vp(FAKE), 4, ctypes.byref(w2), vp(FAKE), vp(FAKE), 8, 16.0, vp(FAKE), vp(0),
                              vp(FAKE), big, vp(0)) == 2
    bargs = lambda dA=FAKE, M=4, H=0, wt=w: (vp(FAKE), vp(FAKE), vp(H), M, ctypes.byref(wt), vp(FAKE), vp(FAKE), 8,
                                           16.0, vp(FAKE), vp(dA), vp(FAKE), vp(FAKE), big, vp(0))
    assert L.qlora_linear_bwd(*bargs(dA=0)) == 1
    assert L.qlora_linear_bwd(*bargs(M=-3)) == 2
    assert L.qlora_linear_bwd(*bargs(H=FAKE + 2)) == 4          # H is read as fp32 words
    assert L.qlora_linear_bwd(*bargs(wt=w2)) == 2


def test_linear_rejects_codes_beyond_32bit_offsets():
    """N*K/2 bytes of codes must be addressable with 32-bit offsets: the largest
    accepted weight has N*K/2 = INT32_MAX rounded down to whole 64-blocks, one more
    row of 64 is rejected, in the forward and the backward alike."""
    L = lib.load()
    vp = ctypes.c_void_p
    big = 1 << 40
    K = 1 << 16
    ok_rows = (2 ** 31 - 1) * 2 // K // 64 * 64          # N*K/2 <= INT32_MAX
    for N, want in ((ok_rows + 64, 2),):
        w = _w(N=N, K=K)
        assert L.qlora_linear_fwd(vp(FAKE), 4, ctypes.byref(w), vp(FAKE), vp(FAKE), 8, 16.0, vp(FAKE), vp(0),
                                  vp(FAKE), big, vp(0)) == want
        assert L.qlora_linear_bwd(vp(FAKE), vp(FAKE), vp(0), 4, ctypes.byref(w), vp(FAKE), vp(FAKE), 8, 16.0,
                                  vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), big, vp(0)) == want
    # the largest accepted size passes validation up to the workspace check
    w = _w(N=ok_rows, K=K)
    assert L.qlora_linear_fwd(vp(FAKE), 4, ctypes.byref(w), vp(FAKE), vp(FAKE), 8, 16.0, vp(FAKE), vp(0),
                              vp(FAKE), 16, vp(0)) == 5


def test_linear_rejects_rows_beyond_32bit_slab_offsets():
    """K and N are each at most 2^23 (the low-rank kernels address 128 rows of X
    or dY with 32-bit byte offsets): 2^23 passes validation up to the workspace
    check, 2^23 + 64 is rejected, for K and for N, forward and backward."""
    L = lib.load()
    vp = ctypes.c_void_p
    big = 1 << 40
    lim = 1 << 23
    for N, K, want in ((64, lim + 64, 2), (lim + 64, 64, 2), (64, lim, 5), (lim, 64, 5)):
        w = _w(N=N, K=K)
        ws = big if want == 2 else 16
        assert L.qlora_linear_fwd(vp(FAKE), 16, ctypes.byref(w), vp(FAKE), vp(FAKE), 8, 16.0, vp(FAKE), vp(0),
                                  vp(FAKE), ws, vp(0)) == want
        assert L.qlora_linear_bwd(vp(FAKE), vp(FAKE), vp(0), 16, ctypes.byref(w), vp(FAKE), vp(FAKE), 8, 16.0,
                                  vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), ws, vp(0)) == want


def test_grouped_forward_rejects_bad_arguments():
    L = lib.load()
    arr = (lib.FwdProblemStruct * 2)()
    for i in range(2):
        arr[i] = lib.FwdProblemStruct(FAKE, 64, _w(N=256, K=512), FAKE, FAKE, 16, 32.0, FAKE, 0)
    vp = ctypes.c_void_p
    assert L.qlora_linear_fwd_grouped(0, arr, vp(FAKE), 1 << 40, vp(0)) == 2
    assert L.qlora_linear_fwd_grouped(9, arr, vp(FAKE), 1 << 40, vp(0)) == 2
    assert L.qlora_linear_fwd_grouped(2, None, vp(FAKE), 1 << 40, vp(0)) == 1
    assert L.qlora_linear_fwd_grouped(2, arr, vp(FAKE), 16, vp(0)) == 5
    assert L.qlora_workspace_size_grouped(2, arr) == 2 * lib.workspace_size(lib.QN_OP_FWD, 64, 256, 512, 16)
    arr[1].r = 65
    assert L.qlora_linear_fwd_grouped(2, arr, vp(FAKE), 1 << 40, vp(0)) == 2
    assert L.qlora_workspace_size_grouped(2, arr) == 0
    arr[1].r = 16
    arr[1].W.K = 500
    assert L.qlora_linear_fwd_grouped(2, arr, vp(FAKE), 1 << 40, vp(0)) == 2


def test_library_fp4_table_equals_oracle_bits():
    """Two derivations of the 4-bit float table from its bit layout (C++ and
    the oracle) give the same fp32 bits."""
    np.testing.assert_array_equal(lib.qn_table("fp4").view(np.uint32), oracle.fp4_table().view(np.uint32))
    np.testing.assert_array_equal(lib.qn_table("nf4").view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_quantize_4bit_and_types_reject_bad_arguments():
    L = lib.load()
    vp = ctypes.c_void_p
    assert L.qn_table(2, (ctypes.c_float * 16)()) == 3
    assert L.qn_table(0, None) == 1
    q = lambda qt=0, aq=0, s2=0: L.qn_quantize_4bit(vp(FAKE), 0, 4, 64, qt, vp(FAKE), vp(FAKE), vp(aq), vp(s2),
                                                    vp(0))
    assert q(qt=2) == 3
    assert q(aq=FAKE) == 1                     # absmax_q without scale2
    assert q(s2=FAKE) == 1
    assert q(aq=FAKE + 2, s2=FAKE) == 4
    w = _w(quant_type=5)
    assert L.nf4_dequant(ctypes.byref(w), vp(FAKE), 0, vp(0)) == 3


def test_adamw8_rejects_bad_arguments():
    L = lib.load()
    vp = ctypes.c_void_p
    ok = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)

    def call(n=64, p=FAKE, aq=FAKE, **kw):
        cfg = lib.AdamWConfigStruct(**dict(ok, **kw))
        return L.qn_adamw8_step(vp(p), vp(FAKE), n, vp(aq), vp(FAKE), vp(FAKE), vp(FAKE), ctypes.byref(cfg), vp(0))
    assert call(p=0) == 1
    assert call(n=0) == 2
    assert call(step=0) == 7
    assert call(beta1=1.0) == 7
    assert call(beta2=-0.1) == 7
    assert call(eps=0.0) == 7
    assert call(lr=float("inf")) == 7
    assert call(p=FAKE + 2) == 4
    assert call(aq=FAKE + 1) == 4
    # well-formed arguments at an address that is neither device memory nor
    # mapped host memory: rejected before any launch
    assert call() == lib.QN_ERR_MEMORY


def test_adamw8_multi_rejects_bad_arguments():
    """Every tensor is checked before anything is launched: a bad tensor
    anywhere in the list (here the last of 40) is reported with the same code
    as the single-tensor call gives it."""
    L = lib.load()
    vp = ctypes.c_void_p
    good = lib.AdamWTensorStruct(FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE)
    ok = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1)

    def call(last=None, count=40, **kw):
        arr = (lib.AdamWTensorStruct * 40)(*([good] * 40))
        if last is not None:
            arr[39] = last
        cfg = lib.AdamWConfigStruct(**dict(ok, **kw))
        return L.qn_adamw8_step_multi(count, arr, ctypes.byref(cfg), vp(0))
    assert L.qn_adamw8_step_multi(1, None, ctypes.byref(lib.AdamWConfigStruct(**ok)), vp(0)) == 1
    assert call(count=0) == 2
    assert call(last=lib.AdamWTensorStruct(0, FAKE, 64, FAKE, FAKE, FAKE, FAKE)) == 1
    assert call(last=lib.AdamWTensorStruct(FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE)) == 2
    assert call(last=lib.AdamWTensorStruct(FAKE + 2, FAKE, 64, FAKE, FAKE, FAKE, FAKE)) == 4
    assert call(last=lib.AdamWTensorStruct(FAKE, FAKE, 64, FAKE + 1, FAKE, FAKE, FAKE)) == 4
    assert call(step=0) == 7
    assert call(eps=-1.0) == 7
    assert call() == lib.QN_ERR_MEMORY
