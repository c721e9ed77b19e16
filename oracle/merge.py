"""Merging a trained adapter into the frozen weight (TEST INFRASTRUCTURE ONLY).

* "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works: Low-Rank
  Adapters": the adapter can be folded into the base weight once, as
  W + (alpha/r) * B @ A; the FAQ: a QLoRA adapter is merged into a
  dequantised (full-precision) copy of the base, not into the 4-bit one.
* "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", "Ship the
  result, and plan for the merge before you need it": merging into the 4-bit
  base would round the sum back onto one of the sixteen rows, and an update
  much smaller than the gap between two rows rounds straight back to the
  original code; the sound route is to merge into a 16-bit copy and save a
  16-bit checkpoint.

So, with w = fl32(table[q] * A_b) the full-precision dequantised weight (the
block scale A_b as in dequantisation, double-quantised or not) and s = alpha/r:

    acc_0 = 0;  acc_j = fl32(acc_{j-1} + B[n, j] * A[j, k]),  j = 1 .. r
    W_m[n, k] = fl32(w[n, k] + fl32(s * acc_r))           (fp32 output)
    W_m16     = bf16(W_m)  (round to nearest even)           (bf16 output)

READINGS (the pages fix the formula, not its arithmetic):
  * the base is the fp32 dequantisation fl32(c * A_b), "restored to full
    precision", not its bf16 rounding;
  * the sum over the rank index runs in fp32 in increasing j; each product of
    two bf16 values is exact in fp32 (8-bit significands), so every step rounds
    once; s multiplies the finished sum, rounded once, and the sum with the
    base is rounded once; no fused operation beyond the exact product;
  * the output is bf16 (the 16-bit checkpoint) or, on request, that fp32 sum.
"""

import numpy as np

from .bf16 import bf16_round
from .nf4 import dequant


def adapter_delta(A, B, alpha):
    """fl32(s * acc_r) with acc summed in fp32 over increasing j, [N, K]."""
    A = np.asarray(A, dtype=np.float32)
    B = np.asarray(B, dtype=np.float32)
    r = A.shape[0]
    if B.shape[1] != r:
        raise ValueError("B is [N, r], A is [r, K]")
    s = np.float32(np.float32(alpha) / np.float32(r))
    acc = np.zeros((B.shape[0], A.shape[1]), dtype=np.float32)
    for j in range(r):
        acc = (acc + (B[:, j:j + 1] * A[j:j + 1, :]).astype(np.float32)).astype(np.float32)
    return (s * acc).astype(np.float32)


def merge(packed, N, K, scale, A, B, alpha, out="bf16", table=None, quant_type="nf4"):
    """The merged weight W_m [N, K]: fp32 values, bf16-rounded when out == "bf16"."""
    w = dequant(packed, N * K, scale, table, quant_type).reshape(N, K)
    m = (w + adapter_delta(A, B, alpha)).astype(np.float32)
    if out == "bf16":
        return bf16_round(m)
    if out == "f32":
        return m
    raise ValueError("out is 'bf16' or 'f32'")
