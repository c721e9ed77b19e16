"""Blockwise 4-bit quantisation, packing and dequantisation (TEST INFRASTRUCTURE ONLY).

Follows "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs":

* "Store a weight in 4 bits ..." -- a 4-bit pattern is the index of a row in a
  16-row table; storing means writing the index of the closest row, reading
  back means looking the row up.
* "The table, and the number that stretches it" -- the worked example: the
  scale of a group is its largest magnitude; dividing by it maps the group into
  [-1, 1]; round to the closest row; multiply the row by the scale to read back.
* "Why the groups are small" -- groups of 64 consecutive weights, each with its
  own scale.
* "What is QLoRA ..." (studyaidesign), "How it actually works" -- N weights at
  b bits take N*b/8 bytes: two 4-bit codes per byte.

READINGS (the pages leave these open):
  * blocks are 64 consecutive elements of the row-major flattening; the last
    block may be partial;
  * "divide every weight by the scale" is carried out as one correctly rounded
    fp32 reciprocal per block, rho = fl32(1/a), then n = fl32(x * rho); where
    that reciprocal does not exist in fp32 (a < 2^-128, 1/a overflows) each
    weight is divided directly, n = fl32(x / a); a block whose absmax is 0
    normalises to all zeros;
  * the closest row is taken in exact arithmetic; an exact tie between two rows
    goes to the LOWER index;
  * element 2i is stored in the low nibble of byte i, element 2i+1 in the high
    nibble; when the element count is odd the unused high nibble is 0;
  * dequantisation is w = fl32(table[q] * A) with A the block's scale (fp32),
    a single fp32 product, no fused operation.
"""

import numpy as np

from .codebook import fp4_table, midpoints, nf4_codebook, sorted_levels

BLOCK = 64


def _flat_f32(w):
    w = np.asarray(w)
    if w.dtype != np.float32:
        raise TypeError("weights must be given as float32 values (bf16 inputs widened exactly)")
    flat = np.ascontiguousarray(w).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite weight: the method does not define a code for it")
    return flat


def n_blocks(n):
    return (n + BLOCK - 1) // BLOCK


def block_absmax(w):
    """a_b = max |x| over elements [64b, 64b+64) of the flattening, fp32[nb]."""
    flat = _flat_f32(w)
    n = flat.size
    nb = n_blocks(n)
    pad = np.zeros(nb * BLOCK, dtype=np.float32)
    pad[:n] = np.abs(flat)
    return pad.reshape(nb, BLOCK).max(axis=1).astype(np.float32)


def normalise(w, absmax):
    """n = fl32(x * fl32(1/a_b)) per element (fl32(x / a_b) where 1/a_b overflows);
    zero where a_b == 0."""
    flat = _flat_f32(w)
    n = flat.size
    a = np.asarray(absmax, dtype=np.float32)
    blk = np.arange(n) // BLOCK
    ab = a[blk]
    safe = np.where(ab > 0, ab, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        rho = (np.float32(1.0) / safe).astype(np.float32)
        out = (flat * rho).astype(np.float32)
    direct = np.isinf(rho)
    if np.any(direct):
        out[direct] = (flat[direct] / safe[direct]).astype(np.float32)
    out[ab == 0] = np.float32(0.0)
    return out


def nearest_code(nrm, table):
    """Index of the closest table row to each fp32 value, ties to the lower index.

    Row i owns the interval (m_{i-1}, m_i] between the exact midpoints, so the
    index is the number of midpoints strictly below the value.
    """
    mids = midpoints(table)
    v = np.asarray(nrm, dtype=np.float32).astype(np.float64)
    return np.searchsorted(mids, v, side="left").astype(np.uint8)


def pack_codes(q):
    """Two 4-bit codes per byte: element 2i low nibble, 2i+1 high nibble."""
    q = np.asarray(q, dtype=np.uint8).reshape(-1)
    if np.any(q > 15):
        raise ValueError("codes are 4-bit")
    n = q.size
    nbytes = (n + 1) // 2
    padded = np.zeros(2 * nbytes, dtype=np.uint8)
    padded[:n] = q
    return (padded[0::2] | (padded[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed, n):
    """Inverse of pack_codes: uint8[n] codes."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(2 * packed.size, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out[:n]


def table_of(quant_type):
    """The 16-entry table (by code) of a 4-bit type: "nf4" or "fp4"."""
    if quant_type == "nf4":
        return nf4_codebook()
    if quant_type == "fp4":
        return fp4_table()
    raise ValueError("quant_type is 'nf4' or 'fp4'")


def quantize(w, table=None, quant_type="nf4"):
    """Blockwise quantisation of a weight array.

    ``table`` (16 values by code) overrides ``quant_type``.  The closest
    distinct value of the table is found with ties to the lower value, then
    written as its code (for a table that is sorted and distinct, like NF4, the
    code is that value's rank).

    Returns (packed uint8[ceil(n/2)], absmax fp32[ceil(n/64)], codes uint8[n]).
    """
    if table is None:
        table = table_of(quant_type)
    flat = _flat_f32(w)
    absmax = block_absmax(flat)
    nrm = normalise(flat, absmax)
    levels, codes_of = sorted_levels(table)
    q = codes_of[nearest_code(nrm, levels)]
    return pack_codes(q), absmax, q


def dequant(packed, n, scale, table=None, quant_type="nf4"):
    """w = fl32(table[q] * A_b) for each element; fp32[n].

    ``scale`` is the per-block fp32 A_b: the absmax itself, or its
    double-quantised reconstruction.
    """
    if table is None:
        table = table_of(quant_type)
    table = np.asarray(table, dtype=np.float32)
    q = unpack_codes(packed, n)
    A = np.asarray(scale, dtype=np.float32)[np.arange(n) // BLOCK]
    return (table[q] * A).astype(np.float32)
