"""The 16-row tables of the 4-bit format (TEST INFRASTRUCTURE ONLY).

NF4 table -- "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs",
sections "Put the rows where the weights are" and "That is NF4": the sixteen
values sit at quantiles of a standard bell curve, are computed once from that
curve (no calibration on the model), one of them is exactly zero, the steps are
finer near zero and coarser in the tails, and after the block scale is divided
out the values span exactly [-1, 1] (section "The table, and the number that
stretches it").

READING (the pages do not give the probabilities):
  * evenly spaced probabilities within each half of the curve, the median
    (p = 1/2) giving the exact zero;
  * the halves are unequal because 16 is even and one row is zero: 7 rows
    below zero (index 0..6), zero at index 7, 8 rows above (index 8..15);
  * the outermost rows cannot sit at p = 0 or 1 (infinite), so they sit at the
    tail probability delta = (1/30 + 1/32)/2 = 31/960: the middle of the
    outermost pile under the two pile counts the text admits (16 piles in the
    "Put the rows where the weights are" recipe, 15 gaps between 16 values);
  * every quantile is divided by z* = Phi^-1(1 - delta) so the table ends at
    exactly -1 and +1; the values are formed in fp64 and rounded to fp32.

Uniform table -- same page, "The table, and the number that stretches it":
sixteen values evenly spread from -1 to 1, gap 2/15.  It is only a fixture for
the page's worked example; it is not part of the product.
"""

from fractions import Fraction
from statistics import NormalDist

import numpy as np

TAIL_DELTA = Fraction(1, 2) * (Fraction(1, 30) + Fraction(1, 32))  # = 31/960
N_NEG = 7   # rows below zero
N_POS = 8   # rows above zero


def nf4_probabilities(delta=TAIL_DELTA):
    """Cumulative probabilities of the 16 rows, as exact Fractions.

    Negative half: delta + i*(1/2 - delta)/7, i = 0..6.  Zero: 1/2.
    Positive half: 1/2 + j*(1/2 - delta)/8, j = 1..8 (j = 8 gives 1 - delta).
    """
    delta = Fraction(delta)
    half = Fraction(1, 2)
    neg = [delta + i * (half - delta) / N_NEG for i in range(N_NEG)]
    pos = [half + j * (half - delta) / N_POS for j in range(1, N_POS + 1)]
    return neg + [half] + pos


def nf4_codebook(delta=TAIL_DELTA):
    """The NF4 table as float32[16] (index 0 = -1, index 7 = 0, index 15 = +1).

    Quantiles come from the standard library's inverse normal CDF (fp64).
    """
    nd = NormalDist()
    probs = nf4_probabilities(delta)
    zstar = nd.inv_cdf(float(1 - Fraction(delta)))
    vals = []
    for k, p in enumerate(probs):
        if k == 0:
            vals.append(-1.0)
        elif k == N_NEG:
            vals.append(0.0)
        elif k == 15:
            vals.append(1.0)
        else:
            vals.append(nd.inv_cdf(float(p)) / zstar)
    return np.array(vals, dtype=np.float64).astype(np.float32)


def uniform_table():
    """Sixteen evenly spaced rows from -1 to 1 (gap 2/15), float32[16].

    Row i is (2i - 15)/15, which is sign-symmetric in fp32.
    """
    return np.array([(2 * i - 15) / 15 for i in range(16)], dtype=np.float64).astype(np.float32)


def fp4_table():
    """The 4-bit floating-point table as float32[16], indexed by code.

    "QLoRA Explained ...", "Turn a LoRA script into a QLoRA script with one
    config object": the library's other 4-bit option is a small floating-point
    layout, not shaped around how weights are distributed, at the same memory;
    the codefinity course page: FP4 uses a floating-point-like structure.

    READING (the pages give no layout): the plainest 4-bit float, one sign bit,
    two exponent bits and one mantissa bit (E2M1, exponent bias 1): for code
    c = s e1 e0 m, exponent field e = 2 e1 + e0,
        e = 0:  (-1)^s * m/2                (0 and 0.5, the subnormals)
        e > 0:  (-1)^s * 2^(e-1) * (1 + m/2)  (1, 1.5, 2, 3, 4, 6)
    divided by the largest magnitude, 6, so that the table spans [-1, 1] like
    the NF4 table (the block scale stretches it the same way); formed in fp64,
    rounded to fp32.  Codes 0 and 8 are +0 and -0: fifteen distinct values.
    """
    vals = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
        vals.append((-1.0 if s else 1.0) * mag / 6.0)
    return np.array(vals, dtype=np.float64).astype(np.float32)


def sorted_levels(table):
    """(distinct values ascending as float32, code of each value).

    Where two codes hold the same value (+0 and -0 of the float table) the
    smaller code is the one a quantiser writes."""
    t = np.asarray(table, dtype=np.float32)
    vals, codes = [], []
    for c in np.argsort(t.astype(np.float64), kind="stable"):
        v = float(t[c])
        if vals and v == vals[-1]:
            codes[-1] = min(codes[-1], int(c))
            continue
        vals.append(v)
        codes.append(int(c))
    return np.array(vals, dtype=np.float32), np.array(codes, dtype=np.uint8)


def midpoints(table):
    """Exact midpoints between neighbouring rows, as fp64[15].

    The rows are fp32 values in [-1, 1]; their sum and its half are exact in
    fp64, so the midpoints carry no rounding.
    """
    t = np.asarray(table, dtype=np.float32).astype(np.float64)
    return (t[:-1] + t[1:]) / 2.0
