"""GPU parity of the fused QLoRA linear (forward and backward) against the fp64 oracle.

Tolerance: relative Frobenius error <= 5e-3 per output tensor (Y, H, dX, dA,
dB), with the adapter term also checked alone (W = 0).  The decode path
(M <= 8) and the MFMA path (M > 8) are both covered, with ragged M, N not a
multiple of the 128-wide tile, several ranks, with and without double
quantisation, and at the full 4096x4096 / 7B-layer / 70B-layer shapes on
sampled output rows.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import REL_FRO_TOL, dev, guarded, guards_intact, host, rel_fro, say, to_dev

pytestmark = pytest.mark.gpu


class Case:
    def __init__(self, N, K, M, r, alpha, seed=0, w_std=0.02, w_zero=False, outliers=False, x_std=1.0,
                 ab_std=0.01):
        self.N, self.K, self.M, self.r, self.alpha = N, K, M, r, alpha
        W = synth.gaussian((N, K), w_std, synth.SEED_W + seed)
        if outliers:
            W = synth.with_outliers(W, 0.001, 10.0)
        if w_zero:
            W = np.zeros((N, K), np.float32)
        self.W = W
        self.Xb = synth.to_bf16(synth.gaussian((M, K), x_std, synth.SEED_X + seed))
        self.Ab = synth.to_bf16(synth.gaussian((r, K), ab_std, synth.SEED_A + seed))
        self.Bb = synth.to_bf16(synth.gaussian((N, r), ab_std, synth.SEED_B + seed))
        self.dYb = synth.to_bf16(synth.gaussian((M, N), 1.0, synth.SEED_DY + seed))
        self.X = synth.bf16_values(self.Xb)
        self.A = synth.bf16_values(self.Ab)
        self.B = synth.bf16_values(self.Bb)
        self.dY = synth.bf16_values(self.dYb)

    def oracle_weight(self, dq=True):
        p, a, _ = oracle.quantize(self.W)
        scale = oracle.dq_absmax(*oracle.double_quant(a)) if dq else a
        return oracle.dequant_bf16_weight(p, self.N, self.K, scale)

    def device(self, dq=True):
        w = lib.quantize_weight(to_dev(self.W), double_quant=True)
        return w, self.Xb.to(dev()), self.Ab.to(dev()), self.Bb.to(dev()), self.dYb.to(dev())


def _check(name, got, ref, tol=REL_FRO_TOL):
    e = rel_fro(got, ref)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:.1e}"
    return e


def run_fwd_bwd(c: Case, dq=True, bwd=True):
    w, X, A, B, dY = c.device()
    Wh = c.oracle_weight(dq)
    Yref, Href = oracle.forward(c.X, Wh, c.A, c.B, c.alpha)
    nY = c.M * c.N * 2
    yf, Y = guarded(nY, torch.bfloat16)
    Y = Y.view(c.M, c.N)
    Y, H = lib.qlora_linear_fwd(X, w, A, B, c.alpha, want_H=True, use_double_quant=dq, Y=Y)
    assert guards_intact(yf, nY), "Y guard band overwritten"
    _check("Y", host(Y), Yref)
    _check("H", host(H), Href)
    if not bwd:
        return
    dXr, dAr, dBr = oracle.backward(c.dY, c.X, Wh, c.A, c.B, c.alpha)
    dX, dA, dB = lib.qlora_linear_bwd(dY, X, w, A, B, c.alpha, use_double_quant=dq)
    _check("dX", host(dX), dXr)
    _check("dA", host(dA), dAr)
    _check("dB", host(dB), dBr)


def test_tiny_config_forward_backward():
    say("tiny config fwd+bwd (decode path, M=4)")
    t = synth.TINY
    run_fwd_bwd(Case(t["N"], t["K"], t["M"], t["r"], t["alpha"]))


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_decode_path_small_M(M):
    say(f"decode path M={M}")
    run_fwd_bwd(Case(256, 512, M, 8, 16.0, seed=M), bwd=(M == 5))


@pytest.mark.parametrize("M,N,K", [(1, 192, 3584), (2, 64, 2560), (3, 320, 6208), (1, 64, 6208), (1, 1024, 8192),
                                   (1, 128, 20480)])
def test_decode_path_ragged(M, N, K):
    """Contraction lengths that are not a multiple of the decode path's
    2048-wide chunk (its out-of-range loads) and that do not fill the last
    K-segment, and ones that do (one and several segments)."""
    say(f"decode path ragged M={M} N={N} K={K}")
    run_fwd_bwd(Case(N, K, M, 16, 32.0, seed=N + K), bwd=False)


@pytest.mark.parametrize("M,N,K", [(1, 192, 3584), (1, 256, 8192), (2, 128, 4096), (3, 320, 6208), (8, 128, 2048)])
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


def _sampled_rows(M, k, seed):
    return np.sort(np.random.default_rng(seed).choice(M, size=min(k, M), replace=False))


def run_full_size_sampled(N, K, M, r, alpha, w_std=0.02, outliers=False, bwd=True, seed=0, rows=64, dq=True):
    """Full-size GPU run; the oracle checks a seeded subset of output rows of Y and
    dX, and dA / dB in full (their reductions over M are cheap in fp64)."""
    c = Case(N, K, M, r, alpha, seed=seed, w_std=w_std, outliers=outliers)
    w, X, A, B, dY = c.device()
    Wh = c.oracle_weight(dq)
    sel = _sampled_rows(M, rows, seed + 1)
    Y, H = lib.qlora_linear_fwd(X, w, A, B, alpha, want_H=True, use_double_quant=dq)
    Yref, Href = oracle.forward(c.X[sel], Wh, c.A, c.B, alpha)
    _check("Y rows", host(Y)[sel], Yref)
    _check("H rows", host(H)[sel], Href)
    if not bwd:
        return
    dX, dA, dB = lib.qlora_linear_bwd(dY, X, w, A, B, alpha, use_double_quant=dq)
    _, dAr, dBr = oracle.backward(c.dY, c.X, None, c.A, c.B, alpha, want_dX=False)
    _check("dA", host(dA), dAr)
    _check("dB", host(dB), dBr)
    dXr, _, _ = oracle.backward(c.dY[sel], c.X[sel], Wh, c.A, c.B, alpha)
    _check("dX rows", host(dX)[sel], dXr)


def test_proj4096_decode_full():
    say("4096x4096 M=1 decode")
    p = synth.PROJ4096
    c = Case(4096, 4096, 1, p["r"], p["alpha"], seed=0)
    w, X, A, B, _ = c.device()
    Y = lib.qlora_linear_fwd(X, w, A, B, c.alpha)
    Yref, _ = oracle.forward(c.X, c.oracle_weight(), c.A, c.B, c.alpha)
    _check("Y", host(Y), Yref)


def test_proj4096_prefill_sampled():
    say("4096x4096 M=2048 prefill fwd+bwd")
    p = synth.PROJ4096
    run_full_size_sampled(4096, 4096, 2048, p["r"], p["alpha"])


def test_proj4096_prefill_fp32_scales_sampled():
    """The same at full size with fp32 block scales (no double quantisation):
    the kernels whose per-step reload is one load shorter."""
    say("4096x4096 M=2048 prefill fwd+bwd, fp32 block scales")
    p = synth.PROJ4096
    run_full_size_sampled(4096, 4096, 2048, p["r"], p["alpha"], seed=11, dq=False)


def test_qwen_layer_shapes_sampled():
    q = synth.QWEN7B
    for name in ("k", "down"):
        N, K = q["linears"][name]
        say(f"qwen {name} {N}x{K} M=4096 fwd+bwd")
        run_full_size_sampled(N, K, q["M"], q["r"], q["alpha"], seed=3, rows=32)


def test_70b_layer_shapes_sampled():
    L = synth.L70B
    N, K = L["linears"]["k"]
    say(f"70b k {N}x{K} M=1 and M=4096 fwd")
    c = Case(N, K, 1, L["r"], L["alpha"], seed=4, w_std=L["w_std"], outliers=True)
    w, X, A, B, _ = c.device()
    Y = lib.qlora_linear_fwd(X, w, A, B, c.alpha)
    Yref, _ = oracle.forward(c.X, c.oracle_weight(), c.A, c.B, c.alpha)
    _check("Y decode", host(Y), Yref)
    run_full_size_sampled(N, K, L["M_prefill"], L["r"], L["alpha"], w_std=L["w_std"], outliers=True,
                          bwd=False, seed=4, rows=32)


def test_qwen_gate_sampled():
    q = synth.QWEN7B
    N, K = q["linears"]["gate"]
    say(f"qwen gate {N}x{K} M=4096 fwd+bwd")
    run_full_size_sampled(N, K, q["M"], q["r"], q["alpha"], seed=5, rows=16)


@pytest.mark.parametrize("name", ["gate", "down"])
def test_70b_large_linears(name):
    """The two largest 70B-layer linears: decode (every output checked) and the
    M=4096 forward on sampled rows; the down projection has the longest
    contraction (28672)."""
    L = synth.L70B
    N, K = L["linears"][name]
    say(f"70b {name} {N}x{K} M=1 and M=4096 fwd")
    c = Case(N, K, 1, L["r"], L["alpha"], seed=6, w_std=L["w_std"], outliers=True)
    w, X, A, B, _ = c.device()
    Wh = c.oracle_weight()
    Y = lib.qlora_linear_fwd(X, w, A, B, c.alpha)
    Yref, _ = oracle.forward(c.X, Wh, c.A, c.B, c.alpha)
    _check("Y decode", host(Y), Yref)
    M = L["M_prefill"]
    Xp = synth.to_bf16(synth.gaussian((M, K), 1.0, synth.SEED_X + 60))
    sel = _sampled_rows(M, 16, 61)
    Yp = lib.qlora_linear_fwd(Xp.to(dev()), w, A, B, c.alpha)
    Yref, _ = oracle.forward(synth.bf16_values(Xp)[sel], Wh, c.A, c.B, c.alpha)
    _check("Y prefill rows", host(Yp)[sel], Yref)
