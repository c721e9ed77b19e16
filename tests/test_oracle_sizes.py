"""The storage totals printed on the pages, from the arrays the oracle returns.

"QLoRA Explained ...", "Shrink the scale factors too, and total up the real
bill"; "What is QLoRA ...", "How it actually works" (N*b/8); the zenaique.com
quiz "Side-by-side" table (saving of about 0.37 bits per parameter).
"""

import numpy as np

import oracle
from oracle import sizes
from tests.conftest import load_golden

G = load_golden("storage_budget.txt")


def _v(name):
    return float(G[name][0]), float(G[name][1])


def _check(name, got):
    v, tol = _v(name)
    assert abs(got - v) <= tol, (name, got, v)


def _arrays_bits(n):
    rng = np.random.default_rng(0)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    packed, absmax, _ = oracle.quantize(w)
    k, step = oracle.double_quant(absmax)
    return 8 * packed.nbytes, 8 * absmax.nbytes, 8 * k.nbytes, 8 * step.nbytes


def test_bits_per_weight_from_actual_arrays():
    n = 16384 * 8                       # whole groups of 256 blocks
    codes, absmax32, k8, step32 = _arrays_bits(n)
    assert codes / n == 4.0
    _check("fp32_scale_bits_per_weight", absmax32 / n)
    _check("fp32_scale_surcharge_frac", (absmax32 / n) / 4.0)
    _check("dq_scale_bits_per_weight", k8 / n)
    _check("dq_group_bits_per_weight", step32 / n)
    total = (codes + k8 + step32) / n
    assert total == 4.126953125
    _check("total_bits_per_weight", total)
    _check("bytes_per_param", total / 8)
    saving = (codes + absmax32) / n - total
    assert saving == 0.373046875
    _check("dq_saving_bits", saving)
    assert saving < _v("dq_saving_upper")[0]
    assert sizes.bits_per_param(n) == total
    assert sizes.bits_per_param(n, double_quant=False) == (codes + absmax32) / n


def test_model_scale_totals():
    bpp = sizes.bits_per_param(16384 * 1024)
    _check("nf4_7b_gb", 7.62e9 * bpp / 8 / 1e9)
    _check("bf16_7b_gb", sizes.memory_bytes(7.62e9, 16) / 1e9)
    assert sizes.memory_bytes(70e9, 0.5) / 1e9 > _v("scales_70b_fp32_gb_min")[0]
    _check("nf4_70b_gb", 70e9 * 0.515625 / 1e9)
    _check("fp16_13b_gb", sizes.memory_bytes(13e9, 16) / 1e9)
    _check("int4_13b_gb", sizes.memory_bytes(13e9, 4) / 1e9)


def test_storage_bytes_match_arrays_on_ragged_shape():
    n = 256 * 512 + 64 * 3 + 5
    rng = np.random.default_rng(1)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    packed, absmax, _ = oracle.quantize(w)
    k, step = oracle.double_quant(absmax)
    assert sizes.storage_bytes(n) == packed.nbytes + k.nbytes + step.nbytes
    assert sizes.storage_bytes(n, double_quant=False) == packed.nbytes + absmax.nbytes
