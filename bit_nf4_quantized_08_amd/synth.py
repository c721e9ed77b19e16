"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and shapes them; it holds none of the
quantisation or layer arithmetic.  Weights are drawn in fp32 from a normal
distribution (trained weights are roughly bell-shaped, "QLoRA Explained ...",
"What a trained model's weights actually look like"); activations and adapters
are drawn in fp32 and converted to bf16 by torch's round-to-nearest-even cast.

Seed convention (numpy ``default_rng``): W = 1, X = 2, A = 3, B = 4, dY = 5,
outlier positions = 6, bulk tile t = 1000 + t.  A caller that needs several
independent draws of one kind adds an offset (``seed + 100 * i``).
"""

import numpy as np

SEED_W, SEED_X, SEED_A, SEED_B, SEED_DY, SEED_OUTLIER = 1, 2, 3, 4, 5, 6
SEED_BULK0 = 1000


def gaussian(shape, std, seed):
    """fp32 array ~ N(0, std^2), from numpy default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def with_outliers(w, frac, factor, seed=SEED_OUTLIER):
    """Multiply a seeded uniform-random subset (frac of the entries) by factor."""
    w = np.array(w, dtype=np.float32, copy=True)
    flat = w.reshape(-1)
    rng = np.random.default_rng(seed)
    k = int(round(frac * flat.size))
    idx = rng.choice(flat.size, size=k, replace=False)
    flat[idx] = (flat[idx] * np.float32(factor)).astype(np.float32)
    return w


def to_bf16(a):
    """CPU torch bf16 tensor of an fp32 array (torch's RNE cast)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_values(t):
    """fp32 numpy values of a bf16 torch tensor (exact widening)."""
    return t.detach().to("cpu").float().numpy()


# Workloads of the pages' shapes.  alpha for the 7B- and 70B-shaped layers keeps
# alpha/r = 2 as in the pages' config (r=16, lora_alpha=32).
TINY = dict(name="tiny", N=256, K=512, M=4, r=8, alpha=16.0, w_std=0.02, x_std=1.0,
            ab_std=0.01, w_dtype="f32")
PROJ4096 = dict(name="proj4096", N=4096, K=4096, r=16, alpha=32.0, w_std=0.02, x_std=1.0,
                ab_std=0.01, M_decode=1, M_prefill=2048)
QWEN7B = dict(name="qwen2.5-7b-layer", M=4096, r=16, alpha=32.0, w_std=0.02,
              linears=dict(q=(3584, 3584), k=(512, 3584), v=(512, 3584), o=(3584, 3584),
                           gate=(18944, 3584), up=(18944, 3584), down=(3584, 18944)))
L70B = dict(name="70b-layer", M_decode=1, M_prefill=4096, r=64, alpha=128.0, w_std=0.015,
            outlier_frac=0.001, outlier_factor=10.0,
            linears=dict(q=(8192, 8192), k=(1024, 8192), v=(1024, 8192), o=(8192, 8192),
                         gate=(28672, 8192), up=(28672, 8192), down=(8192, 28672)))
BULK = dict(name="bulk", tile=(4096, 4096), tiles=454, w_std=0.02)


def tiny_inputs(seed_offset=0):
    """The tiny QLoRA linear: W fp32 [256,512], X/A/B/dY as bf16 tensors."""
    c = TINY
    W = gaussian((c["N"], c["K"]), c["w_std"], SEED_W + seed_offset)
    X = to_bf16(gaussian((c["M"], c["K"]), c["x_std"], SEED_X + seed_offset))
    A = to_bf16(gaussian((c["r"], c["K"]), c["ab_std"], SEED_A + seed_offset))
    B = to_bf16(gaussian((c["N"], c["r"]), c["ab_std"], SEED_B + seed_offset))
    dY = to_bf16(gaussian((c["M"], c["N"]), 1.0, SEED_DY + seed_offset))
    return dict(W=W, X=X, A=A, B=B, dY=dY, r=c["r"], alpha=c["alpha"])
