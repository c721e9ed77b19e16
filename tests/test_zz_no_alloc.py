"""The no-allocation forward (qlora_linear_fwd_noalloc) against qlora_linear_fwd.

Both run the same kernels on the same inputs, so their outputs must agree bit for
bit.  Two calls in a row through the C ABI, the second with a smaller problem
(the static scratch keeps the first call's contents), on the MFMA path and on
the decode path, then the reverse order; a problem whose workspace exceeds the
static scratch is rejected on the host before anything runs.
"""

import ctypes

import numpy as np
import pytest
import torch

from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import dev, say, to_dev

pytestmark = pytest.mark.gpu


def _case(N, K, M, r, seed):
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + seed)
    w = lib.quantize_weight(to_dev(W))
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + seed)).to(dev())
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + seed)).to(dev())
    B = synth.to_bf16(synth.gaussian((N, r), 0.01, synth.SEED_B + seed)).to(dev())
    return w, X, A, B


def _both(w, X, A, B, alpha):
    M, r = X.shape[0], A.shape[0]
    Y0, H0 = lib.qlora_linear_fwd(X, w, A, B, alpha, want_H=True)
    Y1 = torch.full_like(Y0, float("nan"))
    H1 = torch.full_like(H0, float("nan"))
    st = w.struct(True)
    L = lib.load()
    rc = L.qlora_linear_fwd_noalloc(ctypes.c_void_p(X.data_ptr()), M, ctypes.byref(st),
                                    ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()), r,
                                    ctypes.c_float(alpha), ctypes.c_void_p(Y1.data_ptr()),
                                    ctypes.c_void_p(H1.data_ptr()), lib._stream())
    assert rc == 0, lib.status_string(rc)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1), "Y differs from qlora_linear_fwd"
    assert torch.equal(H0, H1), "H differs from qlora_linear_fwd"


@pytest.mark.parametrize("order", ["large_then_small", "decode_then_prefill"])
def test_noalloc_matches_workspace_entry_point(order):
    shapes = {"large_then_small": [(4096, 4096, 2048, 16, 1), (256, 512, 4, 8, 2), (320, 512, 77, 24, 3)],
              "decode_then_prefill": [(28672, 8192, 8, 64, 4), (1024, 8192, 1, 64, 5), (512, 3584, 300, 16, 6)]}
    for N, K, M, r, seed in shapes[order]:
        say(f"noalloc fwd N={N} K={K} M={M} r={r}")
        w, X, A, B = _case(N, K, M, r, seed)
        _both(w, X, A, B, 2.0 * r)


def test_noalloc_rejects_problems_beyond_the_scratch():
    say("noalloc rejects oversize problems")
    need = lib.workspace_size(lib.QN_OP_FWD, 1 << 18, 1024, 1024, 64)
    assert need > lib.QN_NOALLOC_SCRATCH_BYTES
    w = lib.NF4WeightStruct(0x10000, 0x10000, 0, 0, 1024, 1024, 0)
    vp = ctypes.c_void_p
    rc = lib.load().qlora_linear_fwd_noalloc(vp(0x10000), 1 << 18, ctypes.byref(w), vp(0x10000), vp(0x10000), 64,
                                             ctypes.c_float(128.0), vp(0x10000), vp(0), vp(0))
    assert rc == lib.QN_ERR_SCRATCH
