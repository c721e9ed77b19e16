"""GPU parity of the fused QLoRA linear (forward and backward) against the fp64 oracle.

Every output (Y, H, dX, dA, dB) is written into a buffer with guard bands on both
sides, and checked two ways against the oracle:

* relative Frobenius error <= 5e-3 per tensor, and
* element by element, |got - ref| <= 2 * 2^-8 * bound, where bound is the same
  contraction taken over absolute values (for Y: |X| |W_hat|^T + s |H| |B|^T).
  The kernels round each output to bf16 once (2^-9 relative), feed bf16-rounded
  adapter intermediates (s H, dH) to the matrix unit (2^-9 of their share), the
  decode path rounds the table rows rather than their products to bf16 (2^-8),
  and accumulate in fp32; 2 * 2^-8 covers the sum.  A wrong tile, row or
  column shows here even when a norm over the whole tensor would dilute it.

The decode path (M <= 8) and the MFMA path (M > 8) are both covered, with ragged
M, N not a multiple of the 128-wide tile, several ranks, with and without double
quantisation, the backward with the forward's H given and recomputed, and every
linear of the 7B- and 70B-shaped layers at full size (sampled output rows where
the fp64 reference of a whole output would take too long).
"""

import functools

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import REL_FRO_TOL, dev, guarded, guards_intact, host, rel_fro, say, to_dev

pytestmark = pytest.mark.gpu

ELEM_C = 2.0 * 2.0 ** -8


@functools.lru_cache(maxsize=4)
def _weight(N, K, seed, w_std, outliers, w_zero):
    if w_zero:
        return np.zeros((N, K), np.float32)
    W = synth.gaussian((N, K), w_std, synth.SEED_W + seed)
    if outliers:
        W = synth.with_outliers(W, 0.001, 10.0)
    return W


@functools.lru_cache(maxsize=4)
def _oracle_codes(N, K, seed, w_std, outliers, w_zero):
    p, a, _ = oracle.quantize(_weight(N, K, seed, w_std, outliers, w_zero))
    k, step = oracle.double_quant(a)
    return p, a, k, step


class Case:
    def __init__(self, N, K, M, r, alpha, seed=0, w_std=0.02, w_zero=False, outliers=False, x_std=1.0,
                 ab_std=0.01):
        self.N, self.K, self.M, self.r, self.alpha = N, K, M, r, alpha
        self.key = (N, K, seed, w_std, outliers, w_zero)
        self.W = _weight(*self.key)
        self.Xb = synth.to_bf16(synth.gaussian((M, K), x_std, synth.SEED_X + seed))
        self.Ab = synth.to_bf16(synth.gaussian((r, K), ab_std, synth.SEED_A + seed))
        self.Bb = synth.to_bf16(synth.gaussian((N, r), ab_std, synth.SEED_B + seed))
        self.dYb = synth.to_bf16(synth.gaussian((M, N), 1.0, synth.SEED_DY + seed))
        self.X = synth.bf16_values(self.Xb)
        self.A = synth.bf16_values(self.Ab)
        self.B = synth.bf16_values(self.Bb)
        self.dY = synth.bf16_values(self.dYb)
        self.s = alpha / r

    def oracle_weight(self, dq=True):
        p, a, k, step = _oracle_codes(*self.key)
        scale = oracle.dq_absmax(k, step) if dq else a
        return oracle.dequant_bf16_weight(p, self.N, self.K, scale)

    def device(self):
        w = lib.quantize_weight(to_dev(self.W), double_quant=True)
        return w, self.Xb.to(dev()), self.Ab.to(dev()), self.Bb.to(dev()), self.dYb.to(dev())

    def check_codes(self, w):
        """The device codec at this shape is bit-exact with the oracle."""
        p, _, k, step = _oracle_codes(*self.key)
        assert np.array_equal(host(w.codes), p), "codes differ from the oracle"
        assert np.array_equal(host(w.absmax_q), k), "8-bit scales differ from the oracle"
        assert np.array_equal(host(w.scale2).view(np.uint32), step.view(np.uint32)), "group steps differ"


class Out:
    """An output tensor with guard bands on both sides."""

    def __init__(self, shape, dtype):
        self.shape, self.dtype = shape, dtype
        self.nbytes = int(np.prod(shape)) * (2 if dtype == torch.bfloat16 else 4)
        self.full, view = guarded(self.nbytes, dtype)
        self.t = view.view(*shape)

    def check_guards(self, name):
        assert guards_intact(self.full, self.nbytes), f"{name}: guard band overwritten"


def _check(name, got, ref, bound, tol=REL_FRO_TOL):
    """Relative Frobenius error and the elementwise bound (see the module docstring)."""
    got = np.asarray(got, np.float64)
    e = rel_fro(got, ref)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:.1e}"
    err = np.abs(got - ref)
    lim = ELEM_C * np.asarray(bound, np.float64) + 1e-30
    bad = err > lim
    if np.any(bad):
        i = np.unravel_index(int(np.argmax(err / lim)), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} elements beyond the elementwise bound; worst at {i}: "
                             f"got {got[i]!r}, ref {ref[i]!r}, bound {lim[i]!r}")
    return e


def _abs64(a):
    return np.abs(np.asarray(a, np.float64))


def fwd_bounds(c, Wh, X, H):
    return _abs64(X) @ _abs64(Wh).T + c.s * (_abs64(H) @ _abs64(c.B).T)


def check_forward(c, Y, H, Wh, sel=None):
    X = c.X if sel is None else c.X[sel]
    Yref, Href = oracle.forward(X, Wh, c.A, c.B, c.alpha)
    Yg, Hg = host(Y), host(H)
    if sel is not None:
        Yg, Hg = Yg[sel], Hg[sel]
    _check("Y", Yg, Yref, fwd_bounds(c, Wh, X, Href))
    _check("H", Hg, Href, _abs64(X) @ _abs64(c.A).T)


def check_backward(c, dX, dA, dB, Wh, sel=None):
    _, dAr, dBr = oracle.backward(c.dY, c.X, None, c.A, c.B, c.alpha, want_dX=False)
    G, X = _abs64(c.dY), _abs64(c.X)
    Href = np.asarray(c.X, np.float64) @ np.asarray(c.A, np.float64).T
    dHref = c.s * (np.asarray(c.dY, np.float64) @ np.asarray(c.B, np.float64))
    _check("dA", host(dA), dAr, np.abs(dHref).T @ X)
    _check("dB", host(dB), dBr, c.s * (G.T @ np.abs(Href)))
    if dX is None:
        return
    if sel is None:
        dXr, _, _ = oracle.backward(c.dY, c.X, Wh, c.A, c.B, c.alpha)
        got, Gs, dHs = host(dX), G, dHref
    else:
        dXr, _, _ = oracle.backward(c.dY[sel], c.X[sel], Wh, c.A, c.B, c.alpha)
        got, Gs, dHs = host(dX)[sel], G[sel], dHref[sel]
    _check("dX", got, dXr, Gs @ _abs64(Wh) + np.abs(dHs) @ _abs64(c.A))


def run_fwd_bwd(c: Case, dq=True, bwd=True, rows=None, seed=0, check_codes=False):
    """Forward (and backward) on the device, every output guard-banded.  With
    ``rows`` only that many sampled rows of Y, H and dX are compared (dA and dB
    always in full).  The backward runs twice: recomputing H, and with the
    forward's H given; both are checked, and on the MFMA path (where the forward
    and the recompute form H by the same kernel) they must agree bit for bit."""
    w, X, A, B, dY = c.device()
    if check_codes:
        c.check_codes(w)
    Wh = c.oracle_weight(dq)
    sel = None if rows is None else np.sort(np.random.default_rng(seed + 1).choice(c.M, size=min(rows, c.M),
                                                                                   replace=False))
    Y, H = Out((c.M, c.N), torch.bfloat16), Out((c.M, c.r), torch.float32)
    lib.qlora_linear_fwd(X, w, A, B, c.alpha, use_double_quant=dq, Y=Y.t, H=H.t)
    Y.check_guards("Y")
    H.check_guards("H")
    check_forward(c, Y.t, H.t, Wh, sel)
    if not bwd:
        return
    results = []
    for given in (False, True):
        dX, dA, dB = Out((c.M, c.K), torch.bfloat16), Out((c.r, c.K), torch.bfloat16), Out((c.N, c.r), torch.bfloat16)
        lib.qlora_linear_bwd(dY, X, w, A, B, c.alpha, use_double_quant=dq, out=(dX.t, dA.t, dB.t),
                             H=H.t if given else None)
        for name, o in (("dX", dX), ("dA", dA), ("dB", dB)):
            o.check_guards(name + (" (H given)" if given else ""))
        check_backward(c, dX.t, dA.t, dB.t, Wh, sel)
        results.append((dX.t, dA.t, dB.t))
    if c.M > 8:
        for name, a, b in zip(("dX", "dA", "dB"), results[0], results[1]):
            assert torch.equal(a, b), f"{name} differs between a given and a recomputed H"


def test_tiny_config_forward_backward():
    say("tiny config fwd+bwd (decode path, M=4)")
    t = synth.TINY
    run_fwd_bwd(Case(t["N"], t["K"], t["M"], t["r"], t["alpha"]), check_codes=True)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_decode_path_small_M(M):
    say(f"decode path M={M}")
    run_fwd_bwd(Case(256, 512, M, 8, 16.0, seed=M), bwd=(M == 5))


@pytest.mark.parametrize("M,N,K", [(1, 192, 3584), (2, 64, 2560), (3, 320, 6208), (1, 64, 6208), (1, 1024, 8192),
                                   (1, 128, 20480), (8, 192, 6208), (5, 128, 10240)])
def test_decode_path_ragged(M, N, K):
    """Contraction lengths that are not a multiple of the decode path's
    2048-wide chunk (its out-of-range loads) and that do not fill the last
    K-segment, and ones that do (one and several segments)."""
    say(f"decode path ragged M={M} N={N} K={K}")
    run_fwd_bwd(Case(N, K, M, 16, 32.0, seed=N + K), bwd=False)


@pytest.mark.parametrize("M,N,K", [(1, 192, 3584), (1, 256, 8192), (2, 128, 4096), (3, 320, 6208), (8, 128, 2048),
                                   (8, 128, 8192)])
def test_decode_path_fp32_scales(M, N, K):
    """The decode path reading fp32 block scales (no double quantisation),
    with and without a ragged last chunk."""
    say(f"decode path fp32 scales M={M} N={N} K={K}")
    run_fwd_bwd(Case(N, K, M, 16, 32.0, seed=7 * N + K), bwd=False, dq=False)


@pytest.mark.parametrize("M,r", [(1, 1), (2, 7), (1, 64), (8, 40)])
def test_decode_path_ranks(M, r):
    """Adapter ranks that are and are not a multiple of 8 (the decode
    epilogue's vector and scalar reads of B)."""
    say(f"decode path M={M} r={r}")
    run_fwd_bwd(Case(320, 1024, M, r, 2.0 * r, seed=100 + r), bwd=False)


@pytest.mark.parametrize("M,N,r", [(9, 256, 8), (64, 256, 16), (77, 192, 24), (300, 320, 64), (130, 64, 1)])
def test_mfma_path(M, N, r):
    say(f"mfma path M={M} N={N} r={r}")
    run_fwd_bwd(Case(N, 512, M, r, 2.0 * r, seed=M + N))


@pytest.mark.parametrize("K,N", [(64, 128), (128, 64), (192, 192), (320, 128), (256, 320)])
def test_mfma_path_short_contraction(K, N):
    """1 to 5 contraction steps of 64 in the forward (over K) and in dX (over
    N): the pipeline's prologue, its last steps and the adapter step at every
    phase of the stage rotation."""
    say(f"mfma path short contraction K={K} N={N}")
    run_fwd_bwd(Case(N, K, 77, 8, 16.0, seed=K + N))


@pytest.mark.parametrize("M", [4, 200])
def test_adapter_term_alone(M):
    """W = 0: the output is only (alpha/r) (X A^T) B^T, checked on its own scale."""
    say(f"adapter term alone M={M}")
    c = Case(256, 512, M, 16, 32.0, seed=11, w_zero=True, ab_std=0.05)
    run_fwd_bwd(c)


@pytest.mark.parametrize("dq", [False, True])
def test_with_and_without_double_quant(dq):
    say(f"double quant={dq}")
    run_fwd_bwd(Case(256, 1024, 96, 16, 32.0, seed=5, outliers=True), dq=dq)


def test_deterministic():
    say("determinism")
    c = Case(320, 512, 200, 16, 32.0, seed=9)
    w, X, A, B, dY = c.device()
    y1 = lib.qlora_linear_fwd(X, w, A, B, c.alpha)
    y2 = lib.qlora_linear_fwd(X, w, A, B, c.alpha)
    g1 = lib.qlora_linear_bwd(dY, X, w, A, B, c.alpha)
    g2 = lib.qlora_linear_bwd(dY, X, w, A, B, c.alpha)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_proj4096_decode_full():
    say("4096x4096 M=1 decode, every output")
    p = synth.PROJ4096
    run_fwd_bwd(Case(4096, 4096, 1, p["r"], p["alpha"], seed=0), bwd=False, check_codes=True)


def test_proj4096_decode_m8_full():
    """M = 8 (the instance with the most activation registers) over two
    K-segments at 4096x4096, every output."""
    say("4096x4096 M=8 decode, every output")
    p = synth.PROJ4096
    run_fwd_bwd(Case(4096, 4096, 8, p["r"], p["alpha"], seed=0), bwd=False)


def test_proj4096_prefill_sampled():
    say("4096x4096 M=2048 prefill fwd+bwd")
    p = synth.PROJ4096
    run_fwd_bwd(Case(4096, 4096, 2048, p["r"], p["alpha"], seed=0), rows=64, seed=0)


def test_proj4096_prefill_fp32_scales_sampled():
    """The same at full size with fp32 block scales (no double quantisation):
    the kernels whose per-step reload is one load shorter."""
    say("4096x4096 M=2048 prefill fwd+bwd, fp32 block scales")
    p = synth.PROJ4096
    run_fwd_bwd(Case(4096, 4096, 2048, p["r"], p["alpha"], seed=11), dq=False, rows=64, seed=11)


@pytest.mark.parametrize("name", list(synth.QWEN7B["linears"]))
def test_qwen_layer_linear(name):
    """Every linear of the Qwen2.5-7B-shaped layer at M = 4096 tokens, forward
    and backward (sampled rows of Y, H, dX; dA, dB in full; codes bit-exact)."""
    q = synth.QWEN7B
    N, K = q["linears"][name]
    say(f"qwen {name} {N}x{K} M=4096 fwd+bwd")
    seed = 20 + list(q["linears"]).index(name)
    run_fwd_bwd(Case(N, K, q["M"], q["r"], q["alpha"], seed=seed), rows=16, seed=seed, check_codes=True)


@pytest.mark.parametrize("name", list(synth.L70B["linears"]))
def test_70b_layer_linear(name):
    """Every linear of the 70B-shaped layer (N(0, 0.015) weights, 0.1 % outliers
    x10, r = 64): decode at M = 1 with every output checked, and the M = 4096
    forward on sampled rows; codes bit-exact."""
    L = synth.L70B
    N, K = L["linears"][name]
    seed = 40 + list(L["linears"]).index(name)
    say(f"70b {name} {N}x{K} M=1 fwd, every output")
    c = Case(N, K, 1, L["r"], L["alpha"], seed=seed, w_std=L["w_std"], outliers=True)
    run_fwd_bwd(c, bwd=False, check_codes=True)
    say(f"70b {name} {N}x{K} M=4096 fwd, sampled rows")
    cp = Case(N, K, L["M_prefill"], L["r"], L["alpha"], seed=seed, w_std=L["w_std"], outliers=True)
    run_fwd_bwd(cp, bwd=False, rows=12, seed=seed)


def test_70b_gate_decode_m8_full():
    """M = 8 decode over four K-segments of the 70B-shaped gate projection,
    every output."""
    L = synth.L70B
    N, K = L["linears"]["gate"]
    say(f"70b gate {N}x{K} M=8 decode, every output")
    run_fwd_bwd(Case(N, K, 8, L["r"], L["alpha"], seed=44, w_std=L["w_std"], outliers=True), bwd=False)
