"""Storage arithmetic of the format (TEST INFRASTRUCTURE ONLY).

* "What is QLoRA ..." (studyaidesign), "How it actually works": N numbers at
  b bits take N*b/8 bytes.
* "QLoRA Explained ...", "Shrink the scale factors too, and total up the real
  bill": one fp32 scale per 64 weights costs 32/64 bits per weight; stored in
  8 bits it costs 8/64, plus one 32-bit constant per 256 scales (32/16384).

These count the bits of the arrays the quantiser actually returns, so a test
can compare them with the page's totals.
"""

from .dq import GROUP, n_groups
from .nf4 import BLOCK, n_blocks


def storage_bytes(n, double_quant=True):
    """Bytes of codes + scale constants for n weights (block 64, group 256)."""
    codes = (n + 1) // 2
    nb = n_blocks(n)
    if not double_quant:
        return codes + 4 * nb
    return codes + nb + 4 * n_groups(nb)


def bits_per_param(n, double_quant=True):
    return 8.0 * storage_bytes(n, double_quant) / n


def memory_bytes(n_params, bits):
    """N * b / 8."""
    return n_params * bits / 8


__all__ = ["storage_bytes", "bits_per_param", "memory_bytes", "BLOCK", "GROUP"]
