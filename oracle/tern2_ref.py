"""2-bit-aligned dense-ternary comparator format: plain CPU reference.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Sherry paper ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via
Fine-grained Sparsification", Abstract and Figure 2 caption) sets its format
against 2-bit aligned packing, which stores each ternary weight in 2 bits to
keep power-of-two alignment at the cost of wasted bits.  That comparator is
measured on the same ternary matrices.  Reading taken for its layout (the pages
do not give one):
  R8  a weight is a 2-bit two's-complement field: 00 = 0, 01 = +1, 11 = -1
      (10 never produced); 16 weights per little-endian uint32; weight
      4q + p of a word (q, p in 0..3) at bits [8p + 2q, 8p + 2q + 2), so a
      shift by 2q and a mask with 0x03030303 leave four consecutive weights in
      the low bits of the four bytes; row-major, K/16 words per row,
      K % 128 == 0 to share the Sherry shapes.
Products and epilogue are the same as the Sherry reference (R7).
"""
from __future__ import annotations

import numpy as np

from . import sherry_ref

WEIGHTS_PER_WORD = 16
_FIELD = {0: 0, 1: 1, -1: 3}
_VALUE = {0: 0, 1: 1, 3: -1}


def bit_offset(i: int) -> int:
    """Bit offset of weight i (0..15) inside its word: 8 * (i % 4) + 2 * (i // 4)."""
    return 8 * (i % 4) + 2 * (i // 4)


def packed_bytes(n: int, k: int) -> int:
    sherry_ref.check_shape(n, k)
    return n * k // 4


def encode_word(t16) -> int:
    t16 = [int(v) for v in t16]
    if len(t16) != WEIGHTS_PER_WORD or any(v not in _FIELD for v in t16):
        raise ValueError("need 16 ternary weights")
    w = 0
    for i, v in enumerate(t16):
        w |= _FIELD[v] << bit_offset(i)
    return w


def decode_word(w: int) -> list:
    w = int(w)
    out = []
    for i in range(WEIGHTS_PER_WORD):
        f = (w >> bit_offset(i)) & 3
        if f not in _VALUE:
            raise ValueError(f"field 0b10 is not a ternary value (word {w:#010x}, slot {i})")
        out.append(_VALUE[f])
    return out


def pack(t: np.ndarray) -> np.ndarray:
    """int8 ternary [n, k] -> uint32 words [n * k/16]."""
    t = np.asarray(t)
    n, k = t.shape
    sherry_ref.check_shape(n, k)
    if np.any((t != -1) & (t != 0) & (t != 1)):
        raise ValueError("entries must be -1, 0 or +1")
    f = np.where(t < 0, 3, t).astype(np.uint64).reshape(n, k // WEIGHTS_PER_WORD, WEIGHTS_PER_WORD)
    shifts = np.array([bit_offset(i) for i in range(WEIGHTS_PER_WORD)], dtype=np.uint64)
    words = np.bitwise_or.reduce(f << shifts, axis=2)
    return words.astype(np.uint32).reshape(-1)


def pack_weights(w: np.ndarray, scale_dtype=np.float16):
    """Real matrix [n, k] -> (2-bit words, per-row scales).  Reading R8b: the
    ternary matrix and scales are those of the 3:4 quantizer (sherry_ref
    quantize, readings R5/R6), stored in the 2-bit layout R8, so the two
    formats hold the same matrix (the pages compare packings of ternary
    weights and give no separate quantizer for the 2-bit one)."""
    codes, alpha = sherry_ref.quantize(w)
    return pack(sherry_ref.dense_from_codes(codes)), alpha.astype(scale_dtype)


def unpack(words: np.ndarray, n: int, k: int) -> np.ndarray:
    sherry_ref.check_shape(n, k)
    w = np.asarray(words, dtype=np.uint32).reshape(n, k // WEIGHTS_PER_WORD).astype(np.uint64)
    shifts = np.array([bit_offset(i) for i in range(WEIGHTS_PER_WORD)], dtype=np.uint64)
    f = (w[:, :, None] >> shifts) & 3
    if np.any(f == 2):
        raise ValueError("field 0b10 is not a ternary value")
    return np.where(f == 3, -1, f).astype(np.int8).reshape(n, k)


def gemv_i8(words, s_w, n: int, k: int, x: np.ndarray, s_x=None, y_dtype=np.float16):
    t = unpack(words, n, k)
    acc = sherry_ref._exact_int_matmul(t, np.asarray(x).astype(np.int64)).astype(np.int32)
    return acc, sherry_ref.epilogue(acc, s_w, s_x, y_dtype)


def gemm_i8(words, s_w, n: int, k: int, x: np.ndarray, s_x, y_dtype=np.float16):
    t = unpack(words, n, k)
    acc = sherry_ref._exact_int_matmul(np.asarray(x).astype(np.int64), t.T.astype(np.int64)).astype(np.int32)
    return acc, sherry_ref.epilogue(acc, s_w, s_x, y_dtype)
