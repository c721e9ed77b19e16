"""GPU merge (qlora_merge) against the oracle: bit-exact.

The kernel sums the adapter product in the order the definition fixes (fp32,
increasing rank index, exact products), so its fp32 output and the bf16
rounding of it must equal the oracle bit for bit, with and without double
quantisation, for ragged shapes, several ranks, and at full size (every
element of the 4096x4096 projection and of the 70B-shaped k projection;
sampled rows of the 70B-shaped gate projection).  The output is guard-banded.
Also: re-quantising the merged bf16 weight on the device returns the original
codes when the update is small, the loss the pages warn of.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import dev, guarded, guards_intact, host, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(N, K, r, seed, w_std=0.02, b_std=0.01, outliers=False):
    W = synth.gaussian((N, K), w_std, synth.SEED_W + seed)
    if outliers:
        W = synth.with_outliers(W, 0.001, 10.0)
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + seed))
    B = synth.to_bf16(synth.gaussian((N, r), b_std, synth.SEED_B + seed))
    return W, A, B


def _oracle_rows(W, A, B, alpha, dq, out, rows=None):
    N, K = W.shape
    packed, absmax, _ = oracle.quantize(W)
    scale = oracle.dq_absmax(*oracle.double_quant(absmax)) if dq else absmax
    Av, Bv = synth.bf16_values(A), synth.bf16_values(B)
    if rows is None:
        return oracle.merge(packed, N, K, scale, Av, Bv, alpha, out=out)
    res = []
    for n in rows:
        pk = packed[n * K // 2:(n + 1) * K // 2]
        sc = scale[n * K // 64:(n + 1) * K // 64]
        res.append(oracle.merge(pk, 1, K, sc, Av, Bv[n:n + 1], alpha, out=out)[0])
    return np.stack(res)


def _device_merge(W, A, B, alpha, dq, out):
    N, K = W.shape
    w = lib.quantize_weight(to_dev(W))
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    nbytes = N * K * (2 if out == "bf16" else 4)
    full, view = guarded(nbytes, dt)
    res = lib.qlora_merge(w, A.to(dev()), B.to(dev()), alpha, out_dtype=out, use_double_quant=dq,
                          out=view.view(N, K))
    assert guards_intact(full, nbytes), "merge output guard band overwritten"
    return w, res


def _bits(a, out):
    a = np.asarray(a, np.float32)
    return oracle.bf16_bits(a) if out == "bf16" else a.view(np.uint32)


@pytest.mark.parametrize("N,K,r,dq,out", [(256, 512, 8, True, "bf16"), (256, 512, 8, False, "f32"),
                                         (37, 576, 13, True, "f32"), (100, 1088, 1, False, "bf16"),
                                         (64, 64, 64, True, "bf16"), (5, 2112, 40, True, "f32")])
def test_merge_bit_exact(N, K, r, dq, out):
    say(f"merge N={N} K={K} r={r} dq={dq} out={out}")
    W, A, B = _inputs(N, K, r, seed=N + K + r, b_std=0.05)
    _, got = _device_merge(W, A, B, 2.0 * r, dq, out)
    ref = _oracle_rows(W, A, B, 2.0 * r, dq, out)
    g = host(got) if out == "f32" else got.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(g if out == "bf16" else g.view(np.uint32), _bits(ref, out))


def test_merge_full_size():
    """Every element of the 4096x4096 projection (r = 16) and of the 70B-shaped
    k projection (1024 x 8192, r = 64, outliers), sampled rows of the 70B-shaped
    gate projection (28672 x 8192, r = 64)."""
    for (N, K, r, std, outl, rows) in ((4096, 4096, 16, 0.02, False, None), (1024, 8192, 64, 0.015, True, None),
                                      (28672, 8192, 64, 0.015, True, [0, 1, 31, 32, 4097, 28671])):
        say(f"merge full size {N}x{K} r={r}")
        W, A, B = _inputs(N, K, r, seed=N + r, w_std=std, outliers=outl)
        _, got = _device_merge(W, A, B, 2.0 * r, True, "bf16")
        ref = _oracle_rows(W, A, B, 2.0 * r, True, "bf16", rows)
        g = got.view(torch.int16).cpu().numpy().view(np.uint16)
        if rows is not None:
            g = g[rows]
        np.testing.assert_array_equal(g, _bits(ref, "bf16"))


def test_requantised_merge_keeps_the_codes():
    """A small update (B ~ N(0, 1e-4^2)) merged into the bf16 export and
    re-quantised to NF4 on the device comes back as the original codes."""
    say("merge then re-quantise")
    W, A, B = _inputs(1024, 4096, 16, seed=77, b_std=1e-4)
    w, merged = _device_merge(W, A, B, 32.0, True, "bf16")
    codes, _ = lib.nf4_quantize(merged)
    torch.cuda.synchronize()
    assert torch.equal(codes, w.codes)
