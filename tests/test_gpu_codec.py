"""GPU parity of the codec kernels against the oracle: bit-exact.

Quantise (codes, packed bytes, absmax), double quantisation (8-bit codes, fp32
steps) and dequantisation (fp32 and bf16) must equal the oracle's bytes.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import dev, guarded, guards_intact, host, say, to_dev

pytestmark = pytest.mark.gpu


def _gpu_quantize_guarded(W_host, as_bf16):
    """Quantise on the GPU into guard-banded outputs; returns host arrays."""
    N, K = W_host.shape
    n = N * K
    Wd = to_dev(W_host, torch.bfloat16 if as_bf16 else torch.float32)
    cf, codes = guarded((n + 1) // 2, torch.uint8)
    nb = (n + 63) // 64
    af, absmax = guarded(4 * nb, torch.float32)
    lib.nf4_quantize(Wd, codes=codes, absmax=absmax)
    assert guards_intact(cf, (n + 1) // 2), "codes guard band overwritten"
    assert guards_intact(af, 4 * nb), "absmax guard band overwritten"
    return host(codes), host(absmax)


def _oracle_input(W_host, as_bf16):
    if as_bf16:
        return synth.bf16_values(synth.to_bf16(W_host))
    return W_host


SHAPES = [(1, 1), (1, 7), (3, 21), (1, 64), (1, 65), (5, 100), (256, 512), (17, 1000), (64, 4096 + 16)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("as_bf16", [False, True])
def test_quantize_bit_exact(shape, as_bf16):
    say(f"quantize shape={shape} bf16={as_bf16}")
    W = synth.gaussian(shape, 0.02, synth.SEED_W + shape[0] * 7 + shape[1])
    codes, absmax = _gpu_quantize_guarded(W, as_bf16)
    p, a, _ = oracle.quantize(_oracle_input(W, as_bf16))
    np.testing.assert_array_equal(absmax.view(np.uint32), a.view(np.uint32))
    np.testing.assert_array_equal(codes, p)


def test_quantize_edge_values():
    say("quantize edge values")
    c = oracle.nf4_codebook()
    mids = oracle.midpoints(c)
    blocks = []
    b = np.zeros(64, np.float32)                       # zero block
    blocks.append(b)
    b = np.zeros(64, np.float32); b[0] = 1.0           # exact ties at a = 1
    for j, i in enumerate([2, 6, 7, 14]):
        b[1 + 2 * j] = np.float32(mids[i])
        b[2 + 2 * j] = np.nextafter(np.float32(mids[i]), np.float32(np.inf))
        b[20 + 2 * j] = -np.float32(mids[i])
    blocks.append(b)
    b = np.full(64, -0.0, np.float32); b[3] = -2.5      # negative zeros, negative absmax
    blocks.append(b)
    rng = np.random.default_rng(3)
    b = (rng.standard_normal(64) * 1e-39).astype(np.float32)  # subnormal block: 1/a overflows
    blocks.append(b)
    b = (rng.standard_normal(64) * 3e-38).astype(np.float32)  # small normal absmax
    blocks.append(b)
    b = (rng.standard_normal(64) * 2e37).astype(np.float32)   # large magnitudes
    blocks.append(b)
    b = rng.standard_normal(64).astype(np.float32); b[10] = 1e-30  # tiny next to O(1)
    blocks.append(b)
    # every code value reachable: weights exactly at the table rows times a
    b = np.concatenate([c, c * np.float32(0.5), -c, c * np.float32(0.25)]).astype(np.float32) * np.float32(0.37)
    blocks.append(b)
    W = np.concatenate(blocks).reshape(len(blocks), 64)
    for as_bf16 in (False, True):
        Wi = _oracle_input(W, as_bf16)
        codes, absmax = _gpu_quantize_guarded(W, as_bf16)
        p, a, _ = oracle.quantize(Wi)
        np.testing.assert_array_equal(absmax.view(np.uint32), a.view(np.uint32))
        np.testing.assert_array_equal(codes, p)


@pytest.mark.parametrize("nb", [1, 255, 256, 257, 1024 * 5 + 3])
def test_double_quant_bit_exact(nb):
    say(f"double_quant nb={nb}")
    rng = np.random.default_rng(nb)
    a = np.abs(rng.standard_normal(nb) * 0.05).astype(np.float32)
    if nb > 300:
        a[256:512] = 0.0                 # a zero group
        a[600] = 3.0                     # an outlier group
    ad = to_dev(a)
    qf, aq = guarded(nb, torch.uint8)
    sf, s2 = guarded(4 * ((nb + 255) // 256), torch.float32)
    lib.nf4_double_quant(ad, absmax_q=aq, scale2=s2)
    assert guards_intact(qf, nb) and guards_intact(sf, 4 * ((nb + 255) // 256))
    k, step = oracle.double_quant(a)
    np.testing.assert_array_equal(host(s2).view(np.uint32), step.view(np.uint32))
    np.testing.assert_array_equal(host(aq), k)


@pytest.mark.parametrize("shape", [(1, 7), (3, 21), (256, 512), (17, 1000), (130, 4096)])
@pytest.mark.parametrize("dq", [False, True])
def test_dequant_bit_exact(shape, dq):
    say(f"dequant shape={shape} dq={dq}")
    W = synth.with_outliers(synth.gaussian(shape, 0.015, 21), 0.01, 10.0)
    w = lib.quantize_weight(to_dev(W), double_quant=True)
    p, a, _ = oracle.quantize(W)
    n = W.size
    if dq:
        k, step = oracle.double_quant(a)
        scale = oracle.dq_absmax(k, step)
    else:
        scale = a
    ref32 = oracle.dequant(p, n, scale)
    ref16 = oracle.bf16_bits(ref32)
    for fmt in ("f32", "bf16"):
        nbytes = n * (4 if fmt == "f32" else 2)
        of, out = guarded(nbytes, torch.float32 if fmt == "f32" else torch.bfloat16)
        lib.nf4_dequant(w, fmt, use_double_quant=dq, out=out.view(w.N, w.K))
        assert guards_intact(of, nbytes)
        if fmt == "f32":
            np.testing.assert_array_equal(host(out).view(np.uint32), ref32.view(np.uint32))
        else:
            torch.cuda.synchronize()
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(got, ref16)


def test_full_4096_square_round_trip_and_determinism():
    say("quantize+dq+dequant 4096x4096 fp32")
    W = synth.gaussian((4096, 4096), 0.02, synth.SEED_W)
    Wd = to_dev(W)
    w1 = lib.quantize_weight(Wd)
    w2 = lib.quantize_weight(Wd)
    torch.cuda.synchronize()
    assert torch.equal(w1.codes, w2.codes) and torch.equal(w1.absmax_q, w2.absmax_q)
    p, a, _ = oracle.quantize(W)
    k, step = oracle.double_quant(a)
    np.testing.assert_array_equal(host(w1.codes), p)
    np.testing.assert_array_equal(host(w1.absmax).view(np.uint32), a.view(np.uint32))
    np.testing.assert_array_equal(host(w1.absmax_q), k)
    np.testing.assert_array_equal(host(w1.scale2).view(np.uint32), step.view(np.uint32))
    out = lib.nf4_dequant(w1, "f32")
    ref = oracle.dequant(p, W.size, oracle.dq_absmax(k, step))
    np.testing.assert_array_equal(host(out).reshape(-1).view(np.uint32), ref.view(np.uint32))


def test_bulk_bf16_tiles_sampled():
    """Bulk workload tiles (4096x4096 bf16): two seeded tiles, a seeded sample of
    rows checked bit-exactly through quantise, double quant and dequant."""
    for t in (0, 453):
        say(f"bulk tile {t}")
        W = synth.gaussian((4096, 4096), 0.02, synth.SEED_BULK0 + t)
        Wb = synth.to_bf16(W)
        w = lib.quantize_weight(Wb.to(dev()))
        rows = np.random.default_rng(t).choice(4096, 64, replace=False)
        rows.sort()
        Wv = synth.bf16_values(Wb)
        codes = host(w.codes).reshape(4096, 2048)
        absmax = host(w.absmax).reshape(4096, 64)
        for r in rows:
            p, a, _ = oracle.quantize(Wv[r])
            np.testing.assert_array_equal(codes[r], p)
            np.testing.assert_array_equal(absmax[r].view(np.uint32), a.view(np.uint32))
        # double quant over whole groups of 256 blocks (4 rows each) for sampled
        # groups; the oracle's absmax comes from the host input rows
        aq = host(w.absmax_q).reshape(-1)
        s2 = host(w.scale2)
        for g in np.unique(rows // 4):
            _, a_g, _ = oracle.quantize(Wv[4 * g:4 * g + 4])
            k, step = oracle.double_quant(a_g)
            np.testing.assert_array_equal(aq[256 * g:256 * (g + 1)], k)
            assert s2[g] == step[0]
