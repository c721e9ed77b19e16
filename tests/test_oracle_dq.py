"""Pins of the oracle's double quantisation.

"QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", section
"Shrink the scale factors too, and total up the real bill": scales stored in 8
bits, grouped 256 at a time with one 32-bit constant per group.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import dq


def _absmaxes(nb, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(nb * 64) * 0.02).astype(np.float32)
    return oracle.block_absmax(w)


@pytest.mark.parametrize("nb", [1, 255, 256, 257, 1024 + 13])
def test_group_max_gets_top_code_and_error_is_half_step(nb):
    a = _absmaxes(nb, nb)
    k, step = oracle.double_quant(a)
    assert step.size == (nb + 255) // 256 and k.size == nb
    ad = oracle.dq_absmax(k, step)
    for g in range(step.size):
        seg = slice(256 * g, 256 * (g + 1))
        j = 256 * g + int(np.argmax(a[seg]))
        assert k[j] == 255
        err = np.abs(a[seg].astype(np.float64) - ad[seg].astype(np.float64))
        assert np.all(err <= 0.5 * float(step[g]) * (1 + 2e-6) + 1e-30)


def test_brute_force_nearest_grid_point():
    a = _absmaxes(256 * 3, 5)
    k, step = oracle.double_quant(a)
    for b in range(a.size):
        s = Fraction(float(step[b // 256]))
        fa = Fraction(float(a[b]))
        best = min(range(256), key=lambda kk: (abs(fa - kk * s), kk))
        exact_q = fa / s
        near_half = abs(exact_q - (int(exact_q) + Fraction(1, 2))) < Fraction(1, 2 ** 15)
        if near_half:
            assert abs(int(k[b]) - best) <= 1
        else:
            assert int(k[b]) == best


def test_ties_round_down():
    a = np.zeros(256, dtype=np.float32)
    a[0] = 255.0                      # step = 255/255 = 1 exactly
    a[1] = 3.5                        # exact tie -> 3
    a[2] = np.nextafter(np.float32(3.5), np.float32(10))  # -> 4
    a[3] = 0.5                        # tie between 0 and 1 -> 0
    k, step = oracle.double_quant(a)
    assert step[0] == 1.0
    assert list(k[:4]) == [255, 3, 4, 0]


def test_zero_group():
    a = np.zeros(300, dtype=np.float32)
    a[280] = 0.5
    k, step = oracle.double_quant(a)
    assert step[0] == 0 and np.all(k[:256] == 0)
    assert k[280] == 255
    assert np.all(oracle.dq_absmax(k, step)[:256] == 0)


def test_negative_rejected():
    with pytest.raises(ValueError):
        dq.double_quant(np.array([-1.0], dtype=np.float32))
