"""bfloat16 round-to-nearest-even by bit manipulation (TEST INFRASTRUCTURE ONLY).

"QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs", section
"That is NF4": every matrix multiply runs on weights expanded back to bf16;
section "Turn a LoRA script into a QLoRA script with one config object": the
compute dtype named in the config is bf16.

bf16 keeps the top 16 bits of an fp32.  Rounding to nearest, ties to even, on
the dropped 16 bits: add 0x7FFF plus the lowest kept bit, then truncate.
NaN is kept quiet; infinities and overflow to infinity follow from the carry.
"""

import numpy as np


def bf16_bits(x):
    """uint16 bit patterns of RNE(fp32 x)."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    r = r.astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40)), r)
    return (r & np.uint32(0xFFFF)).astype(np.uint16)


def bf16_from_bits(b):
    """fp32 values of bf16 bit patterns (exact widening)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_round(x):
    """RNE(fp32 x) to bf16, returned as fp32 values."""
    return bf16_from_bits(bf16_bits(x))
