"""Sherry 1.25-bit (3:4-sparse ternary) weights on AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libsherry.so (include/sherry.h), built
from the HIP sources in csrc/ by ``ultra_bit_weight_amd.build``; ``sherry`` is
its thin ctypes binding for torch tensors.
"""
__all__ = ["sherry", "build"]
