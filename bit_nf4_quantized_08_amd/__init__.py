"""NF4 blockwise quantisation, double quantisation and the fused QLoRA linear on MI355X.

The compute lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libqlora_nf4.so``, declared in ``include/qlora_nf4.h``).  The Python
layer in :mod:`.lib` only marshals arguments: it hands device pointers, sizes
and the current HIP stream to the library.  PyTorch supplies device memory and
streams.  There is no fallback: if the library is missing, calls raise.

Submodules are imported explicitly (``from bit_nf4_quantized_08_amd import lib``)
so that importing the package itself loads nothing.
"""
