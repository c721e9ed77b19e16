"""Double quantisation of the block scales (TEST INFRASTRUCTURE ONLY).

"QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", section
"Shrink the scale factors too, and total up the real bill": the block scales
are themselves quantised -- each stored in 8 bits, the 8-bit scales grouped 256
at a time with one 32-bit constant per group.

READINGS (the page names neither the 8-bit format nor the 32-bit constant):
  * the stages are independent: weights are coded against the fp32 absmax
    first, then the absmaxes are quantised (the page's order);
  * absmaxes are never negative, so the 8-bit format is an UNSIGNED linear grid
    of 256 levels (a signed grid would waste half its rows, the same waste the
    page counts for the even 4-bit table);
  * the group constant is the grid step: step_g = fl32(c_g / 255) where c_g is
    the largest absmax in the group; groups are 256 consecutive blocks, the
    last one may be partial;
  * k_b is the nearest grid index to the fp32 quotient t = fl32(a_b / step_g),
    ties to the LOWER index (as for the 4-bit rows): k = ceil(t - 1/2), clamped
    to [0, 255];
  * a group whose largest absmax is 0 has step 0 and all k = 0;
  * the reconstructed scale is a'_b = fl32(k_b * step_g).
"""

import numpy as np

GROUP = 256


def n_groups(nb):
    return (nb + GROUP - 1) // GROUP


def double_quant(absmax):
    """Returns (k uint8[nb], step fp32[ng])."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    if np.any(a < 0) or not np.all(np.isfinite(a)):
        raise ValueError("absmax values are finite and non-negative")
    nb = a.size
    ng = n_groups(nb)
    k = np.zeros(nb, dtype=np.uint8)
    step = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        seg = a[g * GROUP:(g + 1) * GROUP]
        c = seg.max() if seg.size else np.float32(0.0)
        s = np.float32(c) / np.float32(255.0)       # fl32 division
        step[g] = s
        if s == 0:
            continue
        t = (seg / s).astype(np.float32)              # fl32 quotient per block
        kk = np.ceil(t.astype(np.float64) - 0.5)      # round half down, exact in fp64
        k[g * GROUP:(g + 1) * GROUP] = np.clip(kk, 0, 255).astype(np.uint8)
    return k, step


def dq_absmax(k, step):
    """a'_b = fl32(k_b * step_g), fp32[nb]."""
    k = np.asarray(k, dtype=np.uint8).reshape(-1)
    step = np.asarray(step, dtype=np.float32).reshape(-1)
    g = np.arange(k.size) // GROUP
    return (k.astype(np.float32) * step[g]).astype(np.float32)

