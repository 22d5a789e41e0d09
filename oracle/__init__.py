"""CPU oracle for the Sherry 1.25-bit ternary format and its products.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The GPU library never uses it,
and this package imports nothing from the GPU library.

Plain, slow, obviously correct: numpy in fp64 (exact integers) with pure-Python
loops kept to the small reference routines.  See ``sherry_ref`` for the 3:4
format, ``tern2_ref`` for the 2-bit dense-ternary comparator, ``tern3_ref``
for the 1.67-bit comparator (three weights in five bits) and ``act_ref`` for
the per-token int8 activation quantization.
"""
from . import act_ref, sherry_ref, tern2_ref, tern3_ref  # noqa: F401
