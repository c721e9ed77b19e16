"""The library's calls enqueue kernels only (no allocation, no synchronisation,
no memset), so they can be captured into a HIP graph.  Replays must reproduce
the eager results exactly, including with eager work and synchronisations of
the program between replays."""

import numpy as np
import pytest
import torch

from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [4, 256])
def test_graph_replays_match_eager(M):
    say(f"graph capture of quantize + forward + backward, M={M}")
    N, K, r, alpha = 512, 1024, 16, 32.0
    W = to_dev(synth.gaussian((N, K), 0.02, 31))
    X = synth.to_bf16(synth.gaussian((M, K), 1.0, 32)).to(dev())
    A = synth.to_bf16(synth.gaussian((r, K), 0.01, 33)).to(dev())
    B = synth.to_bf16(synth.gaussian((N, r), 0.01, 34)).to(dev())
    dY = synth.to_bf16(synth.gaussian((M, N), 1.0, 35)).to(dev())

    w = lib.quantize_weight(W)
    Y_ref = lib.qlora_linear_fwd(X, w, A, B, alpha)
    dX_ref, dA_ref, dB_ref = lib.qlora_linear_bwd(dY, X, w, A, B, alpha)
    torch.cuda.synchronize()

    # Buffers the graph writes into.
    w2 = lib.NF4Weight(torch.empty_like(w.codes), torch.empty_like(w.absmax), torch.empty_like(w.absmax_q),
                       torch.empty_like(w.scale2), N, K)
    Y = torch.empty_like(Y_ref)
    dX, dA, dB = torch.empty_like(dX_ref), torch.empty_like(dA_ref), torch.empty_like(dB_ref)
    ws_f = lib.workspace(lib.QN_OP_FWD, M, N, K, r, dev())
    ws_b = lib.workspace(lib.QN_OP_BWD, M, N, K, r, dev())

    def body():
        lib.nf4_quantize(W, codes=w2.codes, absmax=w2.absmax)
        lib.nf4_double_quant(w2.absmax, absmax_q=w2.absmax_q, scale2=w2.scale2)
        lib.qlora_linear_fwd(X, w2, A, B, alpha, Y=Y, ws=ws_f)
        lib.qlora_linear_bwd(dY, X, w2, A, B, alpha, out=(dX, dA, dB), ws=ws_b)

    body()  # warm the library's one-time host state outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        body()
    for rep in range(3):
        for t in (Y, dX, dA, dB, w2.codes):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        # eager work of the program between replays
        other = lib.qlora_linear_fwd(X, w, A, B, 2.0 * alpha)
        torch.cuda.synchronize()
        assert torch.equal(w2.codes, w.codes), f"replay {rep}: codes"
        assert torch.equal(Y, Y_ref), f"replay {rep}: Y"
        assert torch.equal(dX, dX_ref) and torch.equal(dA, dA_ref) and torch.equal(dB, dB_ref), f"replay {rep}: grads"
        assert not torch.equal(other, Y_ref)


@pytest.mark.parametrize("host_state", [False, True])
def test_graph_replays_adamw8_match_eager(host_state):
    """A captured multi-tensor 8-bit AdamW step (its state in device memory, or
    in pinned host memory) replayed three times equals the same step called
    eagerly on copies, bit for bit after every replay; the placement check runs
    at capture time and the replays reuse its addresses."""
    say(f"graph capture of the multi-tensor AdamW step, host_state={host_state}")
    sizes = [1000, 64, 4096 + 5]
    rng = np.random.default_rng(5)
    pa = [torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16).to(dev())
          for n in sizes]
    pb = [p.clone() for p in pa]
    gs = [torch.from_numpy((rng.standard_normal(n) * 0.05).astype(np.float32)).to(torch.bfloat16).to(dev())
          for n in sizes]
    sa = [lib.AdamW8State(n, dev()) for n in sizes]
    sb = [lib.AdamW8State(n, dev(), host=host_state) for n in sizes]
    hp = dict(lr=1e-3, weight_decay=0.01, step=3)
    lib.adamw8_step_multi(pb, gs, sb, **hp)   # one eager call outside capture on each side
    lib.adamw8_step_multi(pa, gs, sa, **hp)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        lib.adamw8_step_multi(pb, gs, sb, **hp)
    for rep in range(3):
        g.replay()
        lib.adamw8_step_multi(pa, gs, sa, **hp)
        other = torch.ones(1024, device=dev()).sum()   # eager work of the program
        torch.cuda.synchronize()
        assert float(other) == 1024.0
        for i in range(len(sizes)):
            assert torch.equal(pa[i].view(torch.int16), pb[i].view(torch.int16)), f"replay {rep}: param {i}"
            for k in ("m_q", "m_step", "u_q", "u_step"):
                a, b = getattr(sa[i], k).cpu(), getattr(sb[i], k).cpu()
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}: {k} of tensor {i}"
