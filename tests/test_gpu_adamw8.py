"""The 8-bit AdamW step (qn_adamw8_step) against the oracle: bit-exact.

The kernel follows the oracle's fp32 operation order, so parameters, 8-bit
codes and block steps must match bit for bit, step after step (each side fed
its own state), for ragged sizes (partial last block, partial last 256-span)
and with weight decay; parameter and state buffers are guard-banded.
"""

import numpy as np
import pytest
import torch

import oracle.adamw8 as ad
from bit_nf4_quantized_08_amd import lib, synth
from tests.gpu_util import dev, guarded, guards_intact, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 63, 64, 65, 257, 1000, 4096 * 64 + 37])
def test_adamw8_bit_exact_over_steps(n):
    say(f"adamw8 n={n}")
    hp = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    rng = np.random.default_rng(n)
    p0 = synth.bf16_values(synth.to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32)))
    nb = (n + 63) // 64
    pf, pd = guarded(2 * n, torch.bfloat16)
    pd.copy_(torch.from_numpy(p0).to(torch.bfloat16).to(dev()))
    bufs = {k: guarded(b, dt) for k, b, dt in (("m_q", n, torch.int8), ("m_step", 4 * nb, torch.float32),
                                                ("u_q", n, torch.uint8), ("u_step", 4 * nb, torch.float32))}
    st = lib.AdamW8State(n, dev())
    for k in bufs:
        bufs[k][1].zero_()
        setattr(st, k, bufs[k][1])
    mq, ms, uq, us = (np.zeros(n, np.int8), np.zeros(nb, np.float32), np.zeros(n, np.uint8), np.zeros(nb, np.float32))
    p = p0
    for t in range(1, 6):
        g = synth.bf16_values(synth.to_bf16((rng.standard_normal(n) * 0.05 + (p - 0.01)).astype(np.float32)))
        lib.adamw8_step(pd, torch.from_numpy(g).to(torch.bfloat16).to(dev()), st, **hp)
        p, mq, ms, uq, us = ad.adamw8_step(p, g, mq, ms, uq, us, step=t, **hp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(pd).view(np.uint32), p.view(np.uint32), err_msg=f"param, step {t}")
        np.testing.assert_array_equal(host(st.m_q), mq, err_msg=f"m codes, step {t}")
        np.testing.assert_array_equal(host(st.u_q), uq, err_msg=f"u codes, step {t}")
        np.testing.assert_array_equal(host(st.m_step).view(np.uint32), ms.view(np.uint32), err_msg=f"m steps {t}")
        np.testing.assert_array_equal(host(st.u_step).view(np.uint32), us.view(np.uint32), err_msg=f"u steps {t}")
    assert guards_intact(pf, 2 * n), "param guard band overwritten"
    for k, nbytes in (("m_q", n), ("m_step", 4 * nb), ("u_q", n), ("u_step", 4 * nb)):
        assert guards_intact(bufs[k][0], nbytes), f"{k} guard band overwritten"


def test_adamw8_multi_equals_single_calls():
    """qn_adamw8_step_multi over 40 tensors of ragged sizes (two launches of at
    most QN_ADAMW_MULTI tensors) equals qn_adamw8_step on each tensor, bit for
    bit, over three consecutive steps; the tensors' buffers are guard-banded."""
    sizes = [1, 3, 63, 64, 65, 255, 256, 257, 1000, 4096 + 5] * 4
    assert len(sizes) > lib.QN_ADAMW_MULTI
    say(f"adamw8 multi over {len(sizes)} tensors")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-6, weight_decay=0.02)
    rng = np.random.default_rng(77)
    multi, single, guards = [], [], []
    for n in sizes:
        p0 = torch.from_numpy(synth.bf16_values(synth.to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))))
        pf, pd = guarded(2 * n, torch.bfloat16)
        pd.copy_(p0.to(torch.bfloat16).to(dev()))
        guards.append((pf, 2 * n))
        multi.append((pd, lib.AdamW8State(n, dev())))
        single.append((p0.to(torch.bfloat16).to(dev()), lib.AdamW8State(n, dev())))
    for t in range(1, 4):
        grads = [torch.from_numpy(synth.bf16_values(synth.to_bf16(
            (rng.standard_normal(n) * 0.05).astype(np.float32)))).to(torch.bfloat16).to(dev()) for n in sizes]
        lib.adamw8_step_multi([p for p, _ in multi], grads, [s for _, s in multi], step=t, **hp)
        for (p, s), g in zip(single, grads):
            lib.adamw8_step(p, g, s, step=t, **hp)
        torch.cuda.synchronize()
        for i, ((pm, sm), (ps, ss)) in enumerate(zip(multi, single)):
            np.testing.assert_array_equal(host(pm).view(np.uint16), host(ps).view(np.uint16), err_msg=f"param {i} step {t}")
            for k in ("m_q", "u_q", "m_step", "u_step"):
                np.testing.assert_array_equal(host(getattr(sm, k)), host(getattr(ss, k)), err_msg=f"{k} {i} step {t}")
    for pf, nbytes in guards:
        assert guards_intact(pf, nbytes), "param guard band overwritten"


@pytest.mark.parametrize("n", [65, 4096 * 16 + 37])
def test_adamw8_host_state_bit_exact(n):
    """The "paged" placement (QE "Turn a memory spike into a slowdown with a
    paged optimizer"): the 8-bit state in pinned host memory, read and written
    by the kernel across the host link, gives the oracle's parameters and state
    bit for bit, step after step."""
    say(f"adamw8 host-resident state n={n}")
    hp = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    rng = np.random.default_rng(n + 5)
    p0 = synth.bf16_values(synth.to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32)))
    nb = (n + 63) // 64
    pd = torch.from_numpy(p0).to(torch.bfloat16).to(dev())
    st = lib.AdamW8State(n, dev(), host=True)
    for k in ("m_q", "m_step", "u_q", "u_step"):
        t = getattr(st, k)
        assert t.device.type == "cpu" and t.is_pinned(), k
    mq, ms, uq, us = (np.zeros(n, np.int8), np.zeros(nb, np.float32), np.zeros(n, np.uint8), np.zeros(nb, np.float32))
    p = p0
    for t in range(1, 4):
        g = synth.bf16_values(synth.to_bf16((rng.standard_normal(n) * 0.05 + (p - 0.01)).astype(np.float32)))
        lib.adamw8_step(pd, torch.from_numpy(g).to(torch.bfloat16).to(dev()), st, **hp)
        p, mq, ms, uq, us = ad.adamw8_step(p, g, mq, ms, uq, us, step=t, **hp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(pd).view(np.uint32), p.view(np.uint32), err_msg=f"param, step {t}")
        np.testing.assert_array_equal(st.m_q.numpy(), mq, err_msg=f"m codes, step {t}")
        np.testing.assert_array_equal(st.u_q.numpy(), uq, err_msg=f"u codes, step {t}")
        np.testing.assert_array_equal(st.m_step.numpy().view(np.uint32), ms.view(np.uint32), err_msg=f"m steps {t}")
        np.testing.assert_array_equal(st.u_step.numpy().view(np.uint32), us.view(np.uint32), err_msg=f"u steps {t}")


def test_adamw8_multi_mixed_placement_equals_device_state():
    """One multi-tensor step over tensors whose states sit alternately in device
    memory and in pinned host memory equals the same step with every state in
    device memory, bit for bit, over three steps."""
    sizes = [64, 1000, 4096 + 5, 257, 3, 65536]
    say(f"adamw8 multi, mixed state placement, {len(sizes)} tensors")
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.99, eps=1e-6, weight_decay=0.02)
    rng = np.random.default_rng(91)
    pa, pb, sa, sb = [], [], [], []
    for i, n in enumerate(sizes):
        p0 = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(torch.bfloat16).to(dev())
        pa.append(p0.clone())
        pb.append(p0.clone())
        sa.append(lib.AdamW8State(n, dev()))
        sb.append(lib.AdamW8State(n, dev(), host=(i % 2 == 0)))
    for t in range(1, 4):
        gs = [torch.from_numpy((rng.standard_normal(n) * 0.05).astype(np.float32)).to(torch.bfloat16).to(dev())
              for n in sizes]
        lib.adamw8_step_multi(pa, gs, sa, **hp)
        lib.adamw8_step_multi(pb, gs, sb, **hp)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            assert torch.equal(pa[i].view(torch.int16), pb[i].view(torch.int16)), f"param {i}, step {t}"
            for k in ("m_q", "m_step", "u_q", "u_step"):
                a, b = getattr(sa[i], k).cpu(), getattr(sb[i], k).cpu()
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{k} of tensor {i}, step {t}"


def test_adamw8_rejects_pageable_state():
    """State in ordinary (pageable) host memory is out of the kernel's reach:
    both entry points reject it on the host with QN_ERR_MEMORY before any
    launch, and the parameters stay as they were."""
    say("adamw8 pageable state rejected")
    n = 256
    pd = torch.zeros(n, dtype=torch.bfloat16, device=dev())
    gd = torch.ones(n, dtype=torch.bfloat16, device=dev())
    st = lib.AdamW8State(n, dev())
    st.u_step = torch.zeros((n + 63) // 64, dtype=torch.float32)   # pageable host memory
    assert not st.u_step.is_pinned()
    with pytest.raises(lib.QNError) as e:
        lib.adamw8_step(pd, gd, st, lr=1e-2)
    assert e.value.status == lib.QN_ERR_MEMORY
    ok = lib.AdamW8State(n, dev())
    with pytest.raises(lib.QNError) as e:
        lib.adamw8_step_multi([pd, pd.clone()], [gd, gd], [ok, st], lr=1e-2)
    assert e.value.status == lib.QN_ERR_MEMORY
    torch.cuda.synchronize()
    assert not pd.any(), "a rejected call changed the parameters"
