"""One AdamW step on the adapter with 8-bit block-wise state (TEST INFRASTRUCTURE ONLY).

"QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs":
* "Why the groups are small": block-wise quantisation -- blocks of 64 values,
  each with its own scale -- is the same idea that makes 8-bit optimizer state
  work;
* "Turn a LoRA script into a QLoRA script with one config object": the
  optimizer is an 8-bit AdamW (optim="paged_adamw_8bit"); the optimizer state
  belongs to the adapter only;
* "Turn a memory spike into a slowdown with a paged optimizer": the paging is a
  memory-placement valve, not arithmetic (not modelled here).

The update rule is not on the pages.  READING: AdamW as published (Loshchilov
and Hutter, decoupled weight decay), step t >= 1, for parameter p, gradient g:

    m' = b1 m + (1 - b1) g
    v' = b2 v + (1 - b2) g^2
    mh = m' / (1 - b1^t),   vh = v' / (1 - b2^t)
    p' = p - lr (mh / (sqrt(vh) + eps) + wd p)

READINGS for the arithmetic and the 8-bit state (fp32 throughout, every
operation rounded once in this order, no fused operations; the constants
c1 = fl32(1 - b1), c2 = fl32(1 - b2), bc1 = fl32(1 - b1^t), bc2 = fl32(1 - b2^t)
formed in fp64 and rounded once):
    m' = fl(fl(b1 m) + fl(c1 g))
    v' = fl(fl(b2 v) + fl(c2 fl(g g)))
    d  = fl(fl(fl(m'/bc1) / fl(fl(sqrt(fl(v'/bc2))) + eps)) + fl(wd p))
    p' = bf16(fl(p - fl(lr d)))          the adapter stays bf16 (round to nearest even)
  State, per block of 64 consecutive parameters:
    m is stored signed: step_m = fl(max|m'| / 127), k = clamp(ceil(fl(fl(m'/step_m) - 1/2)), -127, 127)
    v is stored through u = fl(sqrt(v')) (same range as m and g): step_u = fl(max u / 255),
      k = clamp(ceil(fl(fl(u/step_u) - 1/2)), 0, 255)
    a zero block has step 0 and codes 0.  Read back: m = fl(k step_m), u = fl(k step_u),
    v = fl(u u).  Initial state: all codes and steps zero.
"""

import numpy as np

from .bf16 import bf16_round

BLOCK = 64


def constants(lr, beta1, beta2, eps, weight_decay, step):
    """The fp32 scalars of step t (bias corrections formed in fp64, rounded once)."""
    f = np.float32
    return dict(lr=f(lr), b1=f(beta1), b2=f(beta2), eps=f(eps), wd=f(weight_decay),
                c1=f(1.0 - float(f(beta1))), c2=f(1.0 - float(f(beta2))),
                bc1=f(1.0 - float(f(beta1)) ** int(step)), bc2=f(1.0 - float(f(beta2)) ** int(step)))


def _blocks(x):
    n = x.size
    nb = (n + BLOCK - 1) // BLOCK
    pad = np.zeros(nb * BLOCK, dtype=np.float32)
    pad[:n] = x
    return pad.reshape(nb, BLOCK)


def quantize_state(x, levels, signed):
    """(codes, step[nb]) of one state array, per block of 64: round the fp32
    quotient x/step to the nearest grid point, ties down, clamped to +-levels
    (signed) or [0, levels]."""
    x = np.asarray(x, dtype=np.float32)
    n = x.size
    B = _blocks(np.abs(x) if signed else x)
    step = (B.max(axis=1) / np.float32(levels)).astype(np.float32)
    per = np.repeat(step, BLOCK)[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(per > 0, (x / np.where(per > 0, per, np.float32(1))).astype(np.float32), np.float32(0))
    k = np.ceil((t - np.float32(0.5)).astype(np.float32))
    lo = -levels if signed else 0
    k = np.clip(k, lo, levels)
    k = np.where(per > 0, k, 0)
    return k.astype(np.int8 if signed else np.uint8), step


def dequantize_state(codes, step):
    codes = np.asarray(codes)
    per = np.repeat(np.asarray(step, dtype=np.float32), BLOCK)[:codes.size]
    return (codes.astype(np.float32) * per).astype(np.float32)


def adamw8_step(p, g, m_q, m_step, u_q, u_step, lr, beta1, beta2, eps, weight_decay, step):
    """One step.  p, g: fp32 values of the bf16 parameters and gradients (flat).
    Returns (p' as fp32 values of bf16, m_q', m_step', u_q', u_step')."""
    c = constants(lr, beta1, beta2, eps, weight_decay, step)
    f = np.float32
    p = np.asarray(p, dtype=np.float32).reshape(-1)
    g = np.asarray(g, dtype=np.float32).reshape(-1)
    m = dequantize_state(m_q, m_step)
    u = dequantize_state(u_q, u_step)
    v = (u * u).astype(f)
    m1 = ((c["b1"] * m).astype(f) + (c["c1"] * g).astype(f)).astype(f)
    v1 = ((c["b2"] * v).astype(f) + (c["c2"] * (g * g).astype(f)).astype(f)).astype(f)
    mh = (m1 / c["bc1"]).astype(f)
    vh = (v1 / c["bc2"]).astype(f)
    den = (np.sqrt(vh).astype(f) + c["eps"]).astype(f)
    d = ((mh / den).astype(f) + (c["wd"] * p).astype(f)).astype(f)
    p1 = bf16_round((p - (c["lr"] * d).astype(f)).astype(f))
    u1 = np.sqrt(v1).astype(f)
    mq, ms = quantize_state(m1, 127, signed=True)
    uq, us = quantize_state(u1, 255, signed=False)
    return p1, mq, ms, uq, us


def adamw_reference(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """Plain AdamW in fp64 with full-precision state: (p', m', v')."""
    p, g, m, v = (np.asarray(a, dtype=np.float64) for a in (p, g, m, v))
    m1 = beta1 * m + (1 - beta1) * g
    v1 = beta2 * v + (1 - beta2) * g * g
    mh = m1 / (1 - beta1 ** step)
    vh = v1 / (1 - beta2 ** step)
    return p - lr * (mh / (np.sqrt(vh) + eps) + weight_decay * p), m1, v1
