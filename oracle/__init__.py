"""CPU oracle for blockwise NF4 quantisation, double quantisation and the QLoRA linear.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct
definition that the HIP library is checked against.  Only the test-suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``bit_nf4_quantized_08_amd``) never imports,
calls or links anything in here, and this package imports nothing from it:
the two share no code, no tables and no constant generators.

Sources (the web pages on QLoRA/NF4 this work is built from):

* "QLoRA Explained: A 4-Bit Base, NF4, and What It Really Costs"
  (skillsuites.com), sections "The table, and the number that stretches it",
  "Why the groups are small", "The two failures that motivate the next
  section", "Put the rows where the weights are", "That is NF4",
  "Shrink the scale factors too, and total up the real bill",
  "Predict the throughput tax before you pay it".
* "LoRA vs QLoRA: Efficient Fine-Tuning Explained" (masterainow.com),
  section "How LoRA Works: Low-Rank Adapters".
* "What is QLoRA, and how does it enable fine-tuning on consumer hardware?"
  (studyaidesign.com), section "How it actually works".
* The zenaique.com QLoRA quiz page, "Side-by-side" table.

Precision: codec steps are carried out in IEEE fp32 exactly where the method
stores fp32 (absmax, reciprocal, normalised weight, products), with decisions
(nearest code, rounding of the 8-bit constants) taken exactly; contractions are
fp64.  Every function states the passage it follows.  Readings of passages the
pages leave open are marked READING in the function docstrings.

Parity status per function:
  codebook.nf4_codebook     pinned (invariants + an independent mpmath
                            derivation); parity against the table shipped by
                            the pages' third-party library: UNPINNED (that
                            table is not available here).
  nf4.quantize / dequant    pinned (pages' worked example, brute force).
  codebook.fp4_table        pinned (the E2M1 values from the bit fields,
                            brute-force nearest value, same storage, worse
                            fit to bell-shaped weights than NF4).
  dq.double_quant           pinned (closed forms, brute force).
  linear.forward / backward pinned (merged-weight identity, finite
                            differences, adjoint identity).
  adamw8.adamw8_step        pinned (first step and trajectory against plain
                            fp64 AdamW, brute-force state rounding, pure weight
                            decay); AdamW itself is a reading (not on the pages).
  merge.merge               pinned (exact rational sum within its rounding
                            bound, zero adapter reads back the dequantised
                            weight, X W_m^T against the forward, re-quantising
                            W_m loses the update as the pages say).
"""

from .codebook import nf4_codebook, uniform_table, midpoints, fp4_table, sorted_levels
from .bf16 import bf16_round, bf16_bits, bf16_from_bits
from .nf4 import quantize, pack_codes, unpack_codes, dequant, block_absmax, table_of
from .dq import double_quant, dq_absmax
from .linear import forward, backward, dequant_bf16_weight
from .merge import merge, adapter_delta
from . import adamw8
from . import sizes

__all__ = [
    "nf4_codebook", "uniform_table", "midpoints", "fp4_table", "sorted_levels", "table_of",
    "bf16_round", "bf16_bits", "bf16_from_bits",
    "quantize", "pack_codes", "unpack_codes", "dequant", "block_absmax",
    "double_quant", "dq_absmax",
    "forward", "backward", "dequant_bf16_weight", "merge", "adapter_delta",
    "sizes", "adamw8",
]
