"""FP4 weights and the fused quantise + double-quant launch on the GPU.

* qn_quantize_4bit with both 4-bit types, fp32 and bf16 sources, with and
  without the fused double quantisation: codes, absmax, 8-bit scales and
  group steps bit-exact with the oracle, for ragged sizes (partial last block,
  partial last 1024-span, partial last group of 16384), and FP4 ties at the
  representable midpoints of its levels.
* FP4 dequantisation bit-exact; the QLoRA forward/backward and the merge with
  FP4 weights against the oracle (same bars as NF4).
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import REL_FRO_TOL, dev, guarded, guards_intact, host, rel_fro, say, to_dev

pytestmark = pytest.mark.gpu

# The last size has more groups of 16384 than the fused kernel has resident
# workgroups (several groups per workgroup), and a partial last group.
SIZES = [(1, 1), (3, 21), (1, 65), (5, 100), (17, 1000), (64, 4096 + 16), (3, 16384 * 2 + 1000), (256, 2048),
         (7, 16384 + 64 * 5 + 3), (2053, 16484)]


def _run(W, qt, bf16, dq):
    N, K = W.shape
    n = N * K
    nb = (n + 63) // 64
    ng = (nb + 255) // 256
    Wd = to_dev(W, torch.bfloat16 if bf16 else torch.float32)
    bufs = {name: guarded(nbytes, dt) for name, nbytes, dt in
            (("codes", (n + 1) // 2, torch.uint8), ("absmax", 4 * nb, torch.float32),
             ("absmax_q", nb, torch.uint8), ("scale2", 4 * ng, torch.float32))}
    w = lib.quantize_4bit(Wd, qt, codes=bufs["codes"][1], absmax=bufs["absmax"][1],
                          absmax_q=bufs["absmax_q"][1] if dq else None, scale2=bufs["scale2"][1] if dq else None,
                          double_quant=dq)
    for name, nbytes in (("codes", (n + 1) // 2), ("absmax", 4 * nb), ("absmax_q", nb), ("scale2", 4 * ng)):
        assert guards_intact(bufs[name][0], nbytes), f"{name} guard band overwritten"
    return w


@pytest.mark.parametrize("shape", SIZES)
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_4bit_bit_exact(shape, qt, bf16):
    say(f"quantize_4bit {qt} shape={shape} bf16={bf16}")
    W = synth.gaussian(shape, 0.02, synth.SEED_W + 31 * shape[0] + shape[1])
    Wo = synth.bf16_values(synth.to_bf16(W)) if bf16 else W
    p, a, _ = oracle.quantize(Wo, quant_type=qt)
    k, step = oracle.double_quant(a)
    for dq in (False, True):
        w = _run(W, qt, bf16, dq)
        np.testing.assert_array_equal(host(w.codes), p)
        np.testing.assert_array_equal(host(w.absmax).view(np.uint32), a.view(np.uint32))
        if dq:
            np.testing.assert_array_equal(host(w.absmax_q), k)
            np.testing.assert_array_equal(host(w.scale2).view(np.uint32), step.view(np.uint32))


def test_fp4_ties_and_levels():
    """Blocks with absmax 1 (so the normalised value is the weight itself)
    holding every FP4 level, the fp32-representable midpoints between levels
    (exact ties: the lower level wins) and their neighbours, and zeros of
    both signs (written as code 0)."""
    say("fp4 ties")
    t = oracle.fp4_table()
    lev = np.unique(t.astype(np.float64))
    mids = [(lev[i] + lev[i + 1]) / 2 for i in range(len(lev) - 1)]
    vals = [1.0] + list(t) + [-0.0]
    for m in mids:
        if np.float32(m) == m:
            vals += [m, np.nextafter(np.float32(m), np.float32(np.inf)), np.nextafter(np.float32(m), np.float32(-np.inf))]
    vals = np.array(vals, np.float32)
    W = np.zeros(((vals.size + 63) // 64) * 64, np.float32)
    W[:vals.size] = vals
    for b in range(W.size // 64):
        W[64 * b] = 1.0
    W = W.reshape(-1, 64)
    p, a, q = oracle.quantize(W, quant_type="fp4")
    w = _run(W, "fp4", False, True)
    np.testing.assert_array_equal(host(w.codes), p)
    assert 8 not in set(q.tolist())


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp4_dequant_bit_exact(out):
    say(f"fp4 dequant {out}")
    W = synth.gaussian((300, 1024), 0.02, 5)
    p, a, _ = oracle.quantize(W, quant_type="fp4")
    scale = oracle.dq_absmax(*oracle.double_quant(a))
    ref = oracle.dequant(p, W.size, scale, quant_type="fp4").reshape(W.shape)
    w = lib.quantize_weight(to_dev(W), quant_type="fp4")
    got = lib.nf4_dequant(w, out)
    if out == "f32":
        np.testing.assert_array_equal(host(got).view(np.uint32), ref.view(np.uint32))
    else:
        np.testing.assert_array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), oracle.bf16_bits(ref))


def test_library_fp4_table_equals_oracle_bits():
    np.testing.assert_array_equal(lib.qn_table("fp4").view(np.uint32), oracle.fp4_table().view(np.uint32))


@pytest.mark.parametrize("M,N,K,r", [(1, 256, 512, 8), (5, 320, 2560, 16), (77, 192, 512, 24), (300, 512, 1024, 64),
                                     (2048, 4096, 4096, 16)])
def test_fp4_linear_forward_backward(M, N, K, r):
    """The decode path (M <= 8) and the MFMA path with FP4 weights against the
    fp64 oracle on the FP4 dequantisation; relative Frobenius <= 5e-3 for Y, H,
    dX, dA, dB (sampled rows of Y and dX at 2048 x 4096)."""
    say(f"fp4 linear M={M} N={N} K={K} r={r}")
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + 9 + N)
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + 9))
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + 9))
    B = synth.to_bf16(synth.gaussian((N, r), 0.01, synth.SEED_B + 9))
    dY = synth.to_bf16(synth.gaussian((M, N), 1.0, synth.SEED_DY + 9))
    alpha = 2.0 * r
    w = lib.quantize_weight(to_dev(W), quant_type="fp4")
    p, a, _ = oracle.quantize(W, quant_type="fp4")
    Wh = oracle.dequant_bf16_weight(p, N, K, oracle.dq_absmax(*oracle.double_quant(a)), quant_type="fp4")
    Xd, Ad, Bd, dYd = (t.to(dev()) for t in (X, A, B, dY))
    Y, H = lib.qlora_linear_fwd(Xd, w, Ad, Bd, alpha, want_H=True)
    dX, dA, dB = lib.qlora_linear_bwd(dYd, Xd, w, Ad, Bd, alpha, H=H)
    Xv, Av, Bv, Gv = (synth.bf16_values(t) for t in (X, A, B, dY))
    sel = np.arange(M) if M <= 512 else np.sort(np.random.default_rng(1).choice(M, 32, replace=False))
    Yr, Hr = oracle.forward(Xv[sel], Wh, Av, Bv, alpha)
    assert rel_fro(host(Y)[sel], Yr) <= REL_FRO_TOL
    assert rel_fro(host(H)[sel], Hr) <= REL_FRO_TOL
    _, dAr, dBr = oracle.backward(Gv, Xv, None, Av, Bv, alpha, want_dX=False)
    dXr, _, _ = oracle.backward(Gv[sel], Xv[sel], Wh, Av, Bv, alpha)
    assert rel_fro(host(dX)[sel], dXr) <= REL_FRO_TOL
    assert rel_fro(host(dA), dAr) <= REL_FRO_TOL
    assert rel_fro(host(dB), dBr) <= REL_FRO_TOL


def test_fp4_merge_bit_exact():
    say("fp4 merge")
    N, K, r = 96, 1024, 16
    W = synth.gaussian((N, K), 0.02, 12)
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, 13))
    B = synth.to_bf16(synth.gaussian((N, r), 0.05, 14))
    w = lib.quantize_weight(to_dev(W), quant_type="fp4")
    got = lib.qlora_merge(w, A.to(dev()), B.to(dev()), 32.0, out_dtype="f32")
    p, a, _ = oracle.quantize(W, quant_type="fp4")
    ref = oracle.merge(p, N, K, oracle.dq_absmax(*oracle.double_quant(a)), synth.bf16_values(A),
                       synth.bf16_values(B), 32.0, out="f32", quant_type="fp4")
    np.testing.assert_array_equal(host(got).view(np.uint32), ref.view(np.uint32))


def _edge_blocks(qt):
    """64-element blocks that take the quantiser's rare paths: zero, every
    element a tie at a representable midpoint, negative zeros, a block whose
    absmax is so small that 1/a overflows fp32 (the oracle then divides each
    weight by a), a small normal absmax, huge magnitudes, a tiny value next to
    O(1) ones."""
    table = oracle.nf4_codebook() if qt == "nf4" else oracle.fp4_table()
    lev = np.unique(table)
    mids = ((lev[:-1].astype(np.float64) + lev[1:]) / 2).astype(np.float32)
    rng = np.random.default_rng(17)
    out = [np.zeros(64, np.float32)]
    b = np.zeros(64, np.float32); b[0] = 1.0
    for j, m in enumerate(mids[:15]):
        b[1 + 2 * j] = m
        b[2 + 2 * j] = np.nextafter(m, np.float32(np.inf))
    out.append(b)
    b = np.full(64, -0.0, np.float32); b[5] = -3.25
    out.append(b)
    out.append((rng.standard_normal(64) * 5e-40).astype(np.float32))
    out.append((rng.standard_normal(64) * 3e-38).astype(np.float32))
    out.append((rng.standard_normal(64) * 2e37).astype(np.float32))
    b = rng.standard_normal(64).astype(np.float32); b[10] = 1e-30
    out.append(b)
    return out


@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("bf16", [False, True])
def test_edge_blocks_inside_full_spans(qt, bf16):
    """The edge blocks placed among ordinary Gaussian blocks inside full
    1024-element spans and full and partial groups of 16384 (the kernels'
    straight-line span path, not only the tail path), plain and with the fused
    double quantisation; bit-exact against the oracle."""
    say(f"edge blocks in full spans {qt} bf16={bf16}")
    N, K = 3, 8192                      # 24 full spans; groups: one full, one partial
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + 901).reshape(-1)
    blocks = _edge_blocks(qt)
    # (block, kind): different lanes and load instructions of a span, both
    # halves of the first group, and the partial second group; the block
    # with an overflowing reciprocal (kind 3) in two spans of its own
    at = [(3, 0), (8, 1), (17, 2), (40, 3), (129, 4), (250, 5), (300, 6), (301, 0), (383, 1), (333, 3)]
    for blk, kind in at:
        W[64 * blk:64 * blk + 64] = blocks[kind]
    W = W.reshape(N, K)
    Wo = synth.bf16_values(synth.to_bf16(W)) if bf16 else W
    p, a, _ = oracle.quantize(Wo, quant_type=qt)
    k, step = oracle.double_quant(a)
    # the blocks of kind 3 really take the division path
    with np.errstate(over="ignore", divide="ignore"):
        assert np.isinf(np.float32(1.0) / a[[40, 333]]).all(), "no block with an overflowing reciprocal"
    for dq in (False, True):
        w = _run(W, qt, bf16, dq)
        np.testing.assert_array_equal(host(w.codes), p)
        np.testing.assert_array_equal(host(w.absmax).view(np.uint32), a.view(np.uint32))
        if dq:
            np.testing.assert_array_equal(host(w.absmax_q), k)
            np.testing.assert_array_equal(host(w.scale2).view(np.uint32), step.view(np.uint32))
