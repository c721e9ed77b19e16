"""Pins of the oracle's NF4 table against what the pages fix.

"QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", sections "Put
the rows where the weights are" and "That is NF4": sixteen values at quantiles
of a standard bell curve, computed once, one of them exactly zero, finer steps
near zero and coarser in the tails than the even table (whose gap is 2/15,
section "The table, and the number that stretches it"), spanning [-1, 1].
"""

import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import codebook as cb


def test_sixteen_rows_span_minus_one_to_one():
    c = cb.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == np.float32(-1.0) and c[15] == np.float32(1.0)
    assert np.all(np.diff(c) > 0)


def test_exact_zero_and_asymmetric_halves():
    c = cb.nf4_codebook()
    assert c[7] == np.float32(0.0)
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_finer_near_zero_coarser_in_tails():
    c = cb.nf4_codebook().astype(np.float64)
    gaps = np.diff(c)
    # moving away from zero, each gap is larger than the previous one
    neg = gaps[:7][::-1]      # gaps from the zero row outwards on the negative side
    pos = gaps[7:]            # gaps from the zero row outwards on the positive side
    assert np.all(np.diff(neg) > 0) and np.all(np.diff(pos) > 0)
    even_gap = 2.0 / 15.0
    assert gaps[6] < even_gap and gaps[7] < even_gap       # next to zero: finer
    assert gaps[0] > even_gap and gaps[14] > even_gap      # outermost: coarser


def _phi(z):
    return 0.5 * math.erfc(-z / math.sqrt(2.0))


def test_rows_sit_at_evenly_spaced_probabilities_per_half():
    """Map the rows back through the normal CDF (math.erfc, not the inverse
    routine the oracle used): equal probability steps within each half."""
    c = cb.nf4_codebook().astype(np.float64)
    delta = float(cb.TAIL_DELTA)
    zstar = math.sqrt(2.0) * float(mpmath.erfinv(1 - 2 * mpmath.mpf(delta)))
    p = np.array([_phi(v * zstar) for v in c])
    assert abs(p[7] - 0.5) < 1e-15
    np.testing.assert_allclose(np.diff(p[:8]), (0.5 - delta) / 7, rtol=0, atol=2e-7)
    np.testing.assert_allclose(np.diff(p[7:]), (0.5 - delta) / 8, rtol=0, atol=2e-7)
    assert abs(p[0] - delta) < 2e-7 and abs(p[15] - (1 - delta)) < 2e-7


def _mp_quantile(p):
    return mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1)


def test_independent_high_precision_derivation_gives_same_fp32_bits():
    """mpmath erfinv at 50 digits, rounded once to fp32, equals the oracle."""
    mpmath.mp.dps = 50
    probs = cb.nf4_probabilities()
    delta = cb.TAIL_DELTA
    zstar = _mp_quantile(mpmath.mpf(1) - mpmath.mpf(delta.numerator) / delta.denominator)
    ref = []
    for k, p in enumerate(probs):
        pm = mpmath.mpf(p.numerator) / p.denominator
        ref.append(float(_mp_quantile(pm) / zstar) if k not in (0, 7, 15) else [-1.0, 0.0, 1.0][(0, 7, 15).index(k)])
    ref32 = np.array(ref, dtype=np.float64).astype(np.float32)
    np.testing.assert_array_equal(ref32.view(np.uint32), cb.nf4_codebook().view(np.uint32))
    # and the fp64 values sit well away from fp32 rounding boundaries, so any
    # accurate fp64 derivation (such as the HIP library's own) rounds the same way
    for v in ref:
        if v in (-1.0, 0.0, 1.0):
            continue
        f = np.float32(v)
        ulp = float(np.spacing(f))
        frac = abs(v - float(f)) / ulp
        assert frac < 0.5 - 0.02, (v, frac)


@pytest.mark.parametrize("delta", [Fraction(1, 32), Fraction(31, 960), Fraction(1, 30)])
def test_invariants_hold_across_tail_readings(delta):
    c = cb.nf4_codebook(delta).astype(np.float64)
    assert c[0] == -1 and c[7] == 0 and c[15] == 1
    assert np.all(np.diff(c) > 0)


def test_uniform_table_gap():
    u = cb.uniform_table().astype(np.float64)
    np.testing.assert_allclose(np.diff(u), 2.0 / 15.0, rtol=0, atol=1e-7)
    assert u[0] == -1 and u[15] == 1
    assert np.all(u != 0)  # an even row count around zero has no zero row
    np.testing.assert_array_equal(u, -u[::-1])


def test_midpoints_are_exact():
    c = cb.nf4_codebook()
    m = cb.midpoints(c)
    for i in range(15):
        assert Fraction(m[i]) == (Fraction(float(c[i])) + Fraction(float(c[i + 1]))) / 2
