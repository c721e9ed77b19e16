"""Pins of the oracle's 8-bit AdamW step.

AdamW itself is not on the pages (a reading: the published rule with decoupled
weight decay); the pages fix the block-wise 8-bit state ("QLoRA Explained ...",
"Why the groups are small") and that the state belongs to the adapter only.
The pins check the step against plain AdamW in fp64 with full-precision state,
the 8-bit state against exact nearest-grid rounding, and the special cases.
"""

from fractions import Fraction

import numpy as np

import oracle.adamw8 as ad

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _zeros(n):
    nb = (n + 63) // 64
    return np.zeros(n, np.int8), np.zeros(nb, np.float32), np.zeros(n, np.uint8), np.zeros(nb, np.float32)


def _bf16(a):
    return ad.bf16_round(np.asarray(a, np.float32))


def test_first_step_matches_plain_adamw():
    """From zero state the first step is plain AdamW's (bias corrections make
    mh = g and vh = g^2, so the move is about lr * sign(g)); the 8-bit state
    plays no part yet.  Within one bf16 rounding of the fp64 rule."""
    rng = np.random.default_rng(0)
    n = 1000
    p = _bf16(rng.standard_normal(n) * 0.01)
    g = _bf16(rng.standard_normal(n) * 0.1)
    p1, *_ = ad.adamw8_step(p, g, *_zeros(n), step=1, **HP)
    ref, _, _ = ad.adamw_reference(p, g, 0 * p, 0 * p, step=1, **HP)
    ulp = np.abs(ref) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(p1 - ref) <= ulp)
    moved = np.abs(g) > 1e-3                 # the move lr * (about 1) exceeds a bf16 step of p
    assert np.all(np.sign(p - p1)[moved] == np.sign(g)[moved])


def test_zero_gradient_is_pure_weight_decay():
    rng = np.random.default_rng(1)
    p = _bf16(rng.standard_normal(130) * 0.05)
    g = np.zeros(130, np.float32)
    p1, mq, ms, uq, us = ad.adamw8_step(p, g, *_zeros(130), step=1, **HP)
    expect = _bf16(p - np.float32(HP["lr"]) * (np.float32(HP["weight_decay"]) * p).astype(np.float32))
    np.testing.assert_array_equal(p1, expect)
    assert not np.any(mq) and not np.any(ms) and not np.any(uq) and not np.any(us)


def test_state_rounding_by_brute_force():
    """Each block's codes are the nearest grid points of step = max/levels to
    the fp32 quotient (exact rational search), ties toward minus infinity,
    the block maximum on the end of the grid, a zero block all zero."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(64 * 3 + 10) * 0.02).astype(np.float32)
    x[64:128] = 0.0
    for levels, signed in ((127, True), (255, False)):
        xs = x if signed else np.abs(x)
        k, step = ad.quantize_state(xs, levels, signed)
        for i, v in enumerate(xs):
            st = step[i // 64]
            if st == 0:
                assert k[i] == 0
                continue
            t = Fraction(float(np.float32(np.float32(v) / st)))
            lo = -levels if signed else 0
            best = min(range(lo, levels + 1), key=lambda j: (abs(Fraction(j) - t), j))
            assert int(k[i]) == best, (levels, i)
        for b in range(len(step)):
            blk = np.abs(k[64 * b:64 * b + 64].astype(np.int32))
            if step[b] > 0:
                assert blk.max() == levels


def test_training_with_8bit_state_tracks_fp64_adamw():
    """A least-squares fit of 512 adapter-sized parameters over 300 steps with
    noisy gradients: the 8-bit optimizer and plain fp64 AdamW both converge,
    to losses within a factor of each other."""
    rng = np.random.default_rng(3)
    n = 512
    target = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p8 = _bf16(np.zeros(n))
    p64 = np.zeros(n)
    m64 = np.zeros(n)
    v64 = np.zeros(n)
    st = _zeros(n)
    hp = dict(HP, lr=2e-3, weight_decay=0.0)
    for t in range(1, 301):
        noise = rng.standard_normal(n) * 0.002
        g8 = _bf16(p8 - target + noise)
        p8, *st = ad.adamw8_step(p8, g8, *st, step=t, **hp)
        p64, m64, v64 = ad.adamw_reference(p64, p64 - target + noise, m64, v64, step=t, **hp)
    l0 = float(np.mean(target.astype(np.float64) ** 2))
    l8 = float(np.mean((p8 - target) ** 2))
    l64 = float(np.mean((p64 - target) ** 2))
    assert l64 < 0.05 * l0 and l8 < 0.05 * l0
    assert l8 < 3 * l64 + 1e-8


def test_state_memory():
    """2 bytes per parameter of codes plus two fp32 steps per 64: 2.125 bytes
    against 8 for fp32 moments."""
    n = 130_000
    mq, ms, uq, us = _zeros(n)
    assert (mq.nbytes + ms.nbytes + uq.nbytes + us.nbytes) / n < 2.126
