"""The QLoRA linear layer, forward and backward, in fp64 (TEST INFRASTRUCTURE ONLY).

* "LoRA vs QLoRA: Efficient Fine-Tuning Explained", "How LoRA Works: Low-Rank
  Adapters": the frozen weight W is d x k, the adapter is B (d x r) times A
  (r x k), and the effective weight is W + (alpha/r) * B @ A.
* "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", "That is
  NF4": the 4-bit base is expanded back to bf16 before every multiply, the
  adapter is bf16 throughout; "Turn a LoRA script into a QLoRA script ...":
  no bias on the adapter.
* Same page, "Name the one memory cost LoRA could not remove" and the
  config section: the frozen base gets no gradient; only the adapter does.

So with W_hat = bf16(dequant(W)) of shape [N, K], X of shape [M, K]:

    H  = X A^T                      [M, r]
    Y  = X W_hat^T + s H B^T        [M, N],  s = alpha / r

and for an upstream gradient G = dL/dY the vector-Jacobian product is

    dH = s G B,  dB = s G^T H,  dA = dH^T X,  dX = G W_hat + dH A.

READINGS: the adapter's dropout is not part of this forward (it is a
training-time random mask, not part of the layer's arithmetic); H is kept
unrounded; every product is taken in fp64 from the exact bf16 input values.
"""

import numpy as np

from .bf16 import bf16_round
from .nf4 import dequant


def dequant_bf16_weight(packed, N, K, scale, table=None, quant_type="nf4"):
    """W_hat = bf16(fl32(table[q] * A_b)) as fp32 values, [N, K]."""
    w = dequant(packed, N * K, scale, table, quant_type)
    return bf16_round(w).reshape(N, K)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def forward(X, W_hat, A, B, alpha):
    """Returns (Y fp64 [M,N], H fp64 [M,r])."""
    X, W_hat, A, B = _f64(X), _f64(W_hat), _f64(A), _f64(B)
    r = A.shape[0]
    s = float(alpha) / float(r)
    H = X @ A.T
    Y = X @ W_hat.T + s * (H @ B.T)
    return Y, H


def backward(G, X, W_hat, A, B, alpha, want_dX=True):
    """Returns (dX [M,K], dA [r,K], dB [N,r]) in fp64; the base gets nothing.

    With want_dX=False (W_hat may then be None) dX is not formed and None is
    returned in its place; dA and dB are unchanged."""
    G, X, A, B = _f64(G), _f64(X), _f64(A), _f64(B)
    r = A.shape[0]
    s = float(alpha) / float(r)
    H = X @ A.T
    dH = s * (G @ B)
    dB = s * (G.T @ H)
    dA = dH.T @ X
    dX = G @ _f64(W_hat) + dH @ A if want_dX else None
    return dX, dA, dB
