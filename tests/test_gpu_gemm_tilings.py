"""Both tilings of the forward dequant-GEMM against the oracle.

The forward picks 256 x 256 tiles for launches with at least two tiles per
compute unit and 256 x 128 tiles otherwise; qn_set_gemm_variant forces any of
the three tilings (256 x 128 with producer waves, 256 x 256 with eight waves
that all multiply and dequantise, 256 x 256 with four such waves).  Each case runs with both forced:
ragged M and N (partial tiles in both directions), 1 to 5 contraction steps
(the pipeline's prologue and the adapter step at both stage parities), ranks
1 to 64, fp32 and 8-bit block scales, both 4-bit types, and a grouped launch.
Y and H: relative Frobenius <= 5e-3 against the fp64 oracle and the
elementwise bound, Y guard-banded; the two tilings also agree with each other
within that bound.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import REL_FRO_TOL, dev, guarded, guards_intact, host, rel_fro, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_variant():
    yield
    lib.set_gemm_variant(0)


def _case(M, N, K, r, seed, qt="nf4", dq=True):
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + seed)
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + seed))
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + seed))
    B = synth.to_bf16(synth.gaussian((N, r), 0.02, synth.SEED_B + seed))
    w = lib.quantize_weight(to_dev(W), quant_type=qt)
    p, a, _ = oracle.quantize(W, quant_type=qt)
    scale = oracle.dq_absmax(*oracle.double_quant(a)) if dq else a
    Wh = oracle.dequant_bf16_weight(p, N, K, scale, quant_type=qt)
    return w, X, A, B, Wh


def _fwd(w, X, A, B, alpha, dq):
    M, N = X.shape[0], w.N
    full, Y = guarded(M * N * 2, torch.bfloat16)
    Y = Y.view(M, N)
    Y, H = lib.qlora_linear_fwd(X.to(dev()), w, A.to(dev()), B.to(dev()), alpha, Y=Y, want_H=True,
                                use_double_quant=dq)
    assert guards_intact(full, M * N * 2), "Y guard band overwritten"
    return host(Y), host(H)


def _check(Y, H, X, A, B, Wh, alpha):
    Xv, Av, Bv = (synth.bf16_values(t) for t in (X, A, B))
    Yr, Hr = oracle.forward(Xv, Wh, Av, Bv, alpha)
    assert rel_fro(Y, Yr) <= REL_FRO_TOL
    assert rel_fro(H, Hr) <= REL_FRO_TOL
    s = alpha / A.shape[0]
    bound = np.abs(Xv.astype(np.float64)) @ np.abs(Wh.astype(np.float64)).T + s * np.abs(Hr) @ np.abs(Bv).T
    assert np.all(np.abs(Y - Yr) <= 2 * 2.0 ** -8 * bound + 1e-30)


@pytest.mark.parametrize("M,N,K,r,qt,dq", [
    (300, 320, 512, 16, "nf4", True),
    (77, 192, 64, 8, "nf4", True),       # one contraction step
    (257, 256, 128, 64, "nf4", False),   # two steps, fp32 scales
    (513, 576, 192, 24, "fp4", True),    # three steps
    (256, 64, 256, 1, "nf4", True),
    (130, 448, 320, 40, "nf4", False),   # five steps
    (1024, 1024, 2048, 16, "nf4", True),
])
def test_both_tilings_match_the_oracle(M, N, K, r, qt, dq):
    w, X, A, B, Wh = _case(M, N, K, r, seed=M + N + K, qt=qt, dq=dq)
    out = {}
    for v in (1, 2, 3):
        say(f"tiling {v}: M={M} N={N} K={K} r={r} {qt} dq={dq}")
        lib.set_gemm_variant(v)
        out[v] = _fwd(w, X, A, B, 2.0 * r, dq)
        _check(*out[v], X, A, B, Wh, 2.0 * r)


@pytest.mark.parametrize("variant", [1, 2, 3])
def test_grouped_launch_equals_single_calls(variant):
    """A grouped launch of three problems on each tiling equals the single
    calls on it bit for bit, and the oracle within the bars.  The group's K
    (512, 256, 192) is not all a multiple of 256, so the group loads block
    scales every step, while the single calls with K = 512 and 256 load them
    four steps at a time: the two scale paths must agree exactly."""
    lib.set_gemm_variant(variant)
    cases = [_case(300, 320, 512, 16, seed=1), _case(700, 1024, 256, 64, seed=2), _case(65, 64, 192, 8, seed=3)]
    items, outs = [], []
    for (w, X, A, B, Wh) in cases:
        M, N = X.shape[0], w.N
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        H = torch.empty((M, A.shape[0]), dtype=torch.float32, device=dev())
        items.append((X.to(dev()), w, A.to(dev()), B.to(dev()), 2.0 * A.shape[0], Y, H))
    say(f"tiling {variant} grouped")
    lib.FwdGroup(items).run()
    torch.cuda.synchronize()
    for (X, w, A, B, alpha, Y, H), (_, Xh, Ah, Bh, Wh) in zip(items, cases):
        Y1, H1 = lib.qlora_linear_fwd(X, w, A, B, alpha, want_H=True)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y1) and torch.equal(H, H1)
        _check(host(Y), host(H), Xh, Ah, Bh, Wh, alpha)


@pytest.mark.parametrize("M,N,K,r,qt,dq", [
    (300, 320, 512, 16, "nf4", True),    # ragged M; five contraction steps over N
    (77, 64, 192, 8, "nf4", True),       # one step; a partial 256-wide column tile
    (513, 576, 320, 24, "nf4", False),   # fp32 scales; nine steps
    (256, 128, 256, 1, "nf4", True),     # rank 1
    (200, 256, 512, 16, "fp4", True),
    (1024, 1024, 2048, 64, "nf4", True),
])
def test_dx_tilings_match_the_oracle(M, N, K, r, qt, dq):
    """The backward's dX = dY W_hat + dH A on both tilings (256 x 128 and
    256 x 256, forced) against the fp64 oracle: relative Frobenius <= 5e-3 and
    the elementwise bound |err| <= 2^-7 (|dY| |W_hat| + |dH| |A|), dX
    guard-banded; dA and dB do not depend on the tiling."""
    w, X, A, B, Wh = _case(M, N, K, r, seed=M + 3 * N + K, qt=qt, dq=dq)
    dY = synth.to_bf16(synth.gaussian((M, N), 1.0, synth.SEED_X + 77 + M))
    Xv, Av, Bv, Gv = (synth.bf16_values(t) for t in (X, A, B, dY))
    alpha = 2.0 * r
    dXr, _, _ = oracle.backward(Gv, Xv, Wh, Av, Bv, alpha)
    dH = (alpha / r) * (Gv.astype(np.float64) @ Bv.astype(np.float64))
    bound = np.abs(Gv.astype(np.float64)) @ np.abs(Wh.astype(np.float64)) + np.abs(dH) @ np.abs(Av.astype(np.float64))
    out = {}
    for v in (1, 2):
        say(f"dX tiling {v}: M={M} N={N} K={K} r={r} {qt} dq={dq}")
        lib.set_gemm_variant(v)
        full, dX = guarded(M * K * 2, torch.bfloat16)
        dX = dX.view(M, K)
        dA = torch.empty((r, K), dtype=torch.bfloat16, device=dev())
        dB = torch.empty((N, r), dtype=torch.bfloat16, device=dev())
        lib.qlora_linear_bwd(dY.to(dev()), X.to(dev()), w, A.to(dev()), B.to(dev()), alpha, use_double_quant=dq,
                             out=(dX, dA, dB))
        torch.cuda.synchronize()
        assert guards_intact(full, M * K * 2), "dX guard band overwritten"
        got = host(dX)
        assert rel_fro(got, dXr) <= REL_FRO_TOL
        assert np.all(np.abs(got - dXr) <= 2 * 2.0 ** -8 * bound + 1e-30)
        out[v] = got
    assert np.all(np.abs(out[1] - out[2]) <= 2 * 2.0 ** -8 * bound + 1e-30)


@pytest.mark.parametrize("variant", [1, 2, 3])
def test_tilings_repeat_exactly(variant):
    """Four repetitions of a forward over more than a thousand tiles (and, on
    the tilings dX has, of a backward whose dX covers hundreds of tiles) give
    identical bits.  Each tile stages activation slabs with direct-to-LDS loads
    that a barrier must wait for (in the prologue, and on the 256 x 128 tiling
    in the last half-step of an odd step count, which K = 320 gives); a tile
    that read a slab early would show up as differing rows in some
    repetition."""
    lib.set_gemm_variant(variant)
    K = 320 if variant == 1 else 512
    say(f"tiling {variant}: repeated forward 4096 x 18944 x {K}")
    M, N, r = 4096, 18944, 16
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + 91)
    w = lib.quantize_weight(to_dev(W))
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + 91)).to(dev())
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + 91)).to(dev())
    B = synth.to_bf16(synth.gaussian((N, r), 0.02, synth.SEED_B + 91)).to(dev())
    ys = [lib.qlora_linear_fwd(X, w, A, B, 2.0 * r) for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(1, 4):
        assert torch.equal(ys[i], ys[0]), f"forward repetition {i} differs"
    del ys, w, X, A, B
    if variant == 3:
        return
    N = 320 if variant == 1 else 512
    say(f"tiling {variant}: repeated backward, dX 4096 x 8192 from N = {N}")
    M, K, r = 4096, 8192, 16
    W = synth.gaussian((N, K), 0.02, synth.SEED_W + 92)
    w = lib.quantize_weight(to_dev(W))
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + 92)).to(dev())
    dY = synth.to_bf16(synth.gaussian((M, N), 1.0, synth.SEED_X + 93)).to(dev())
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, synth.SEED_A + 92)).to(dev())
    B = synth.to_bf16(synth.gaussian((N, r), 0.02, synth.SEED_B + 92)).to(dev())
    gs = [lib.qlora_linear_bwd(dY, X, w, A, B, 2.0 * r) for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(1, 4):
        assert all(torch.equal(a, b) for a, b in zip(gs[i], gs[0])), f"backward repetition {i} differs"
