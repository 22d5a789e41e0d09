"""1.67-bit comparator (three ternary weights in five bits): plain CPU reference.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library.

The Sherry paper ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization
via Fine-grained Sparsification") sets its format against two others: 2-bit
aligned packing, and a 1.67-bit strategy that packs three ternary weights into
five bits (Abstract: irregular packing that slows inference; Figure 2
caption, middle: SIMD-unfriendly 3-way patterns).  Three ternary weights take
3^3 = 27 values, which fit five bits.  Readings taken for the layout:
  F1  a code holds three consecutive weights of a row along K:
      c = (t0 + 1) + 3 (t1 + 1) + 9 (t2 + 1), 0 .. 26 (27 .. 31 unused);
  F2  32 codes (96 weights) form a group of five little-endian uint32 words,
      one LSB-first bitstream: code j at bits [5j, 5j + 5) (as the 3:4 format);
  F3  a row's K weights are padded with zeros to K3 = 96 ceil(K / 96), i.e.
      G3 = K3 / 96 groups, stored in the two-part row layout of the 3:4 format:
      words 0-3 of group g at word 4g, word 4 at word 4 G3 + g;
  F4  K % 128 == 0, as for the other formats (x is int8 in 16-byte units).
A row of K = 2048 weights takes 22 groups (110 words, 1.72 bits per weight);
K = 8192 takes 86 groups (1.68 bits per weight).
"""
from __future__ import annotations

import numpy as np

GROUP_W = 96   # weights per group
GROUP_CODES = 32


def groups(k: int) -> int:
    return -(-k // GROUP_W)


def check_shape(n: int, k: int) -> None:
    if n <= 0 or k <= 0 or k % 128 != 0:
        raise ValueError("n, k must be positive and k a multiple of 128")


def packed_words(n: int, k: int) -> int:
    check_shape(n, k)
    return n * 5 * groups(k)


def encode_block(t3) -> int:
    """F1: three ternary weights -> code 0 .. 26."""
    t0, t1, t2 = (int(v) for v in t3)
    for v in (t0, t1, t2):
        if v not in (-1, 0, 1):
            raise ValueError("weights must be ternary")
    return (t0 + 1) + 3 * (t1 + 1) + 9 * (t2 + 1)


def decode_block(c: int) -> tuple:
    """F1 inverted: code 0 .. 26 -> (t0, t1, t2)."""
    if not 0 <= c < 27:
        raise ValueError("code out of range")
    return (c % 3 - 1, (c // 3) % 3 - 1, c // 9 - 1)


def pack(t: np.ndarray) -> np.ndarray:
    """Dense ternary T [n, k] -> packed words (F1-F4), row by row."""
    t = np.asarray(t)
    n, k = t.shape
    check_shape(n, k)
    G = groups(k)
    padded = np.zeros((n, G * GROUP_W), dtype=np.int64)
    padded[:, :k] = t
    out = np.zeros((n, 5 * G), dtype=np.uint32)
    for r in range(n):
        for g in range(G):
            stream = 0
            for j in range(GROUP_CODES):
                w0 = GROUP_W * g + 3 * j
                stream |= encode_block(padded[r, w0:w0 + 3]) << (5 * j)
            for i in range(5):
                word = (stream >> (32 * i)) & 0xFFFFFFFF
                out[r, 4 * g + i if i < 4 else 4 * G + g] = word
    return out.reshape(-1)


def unpack(words: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed words -> dense int8 T [n, k] (the padding is dropped)."""
    check_shape(n, k)
    G = groups(k)
    w = np.asarray(words, dtype=np.uint32).reshape(n, 5 * G)
    t = np.zeros((n, G * GROUP_W), dtype=np.int8)
    for r in range(n):
        for g in range(G):
            parts = [int(w[r, 4 * g + i]) for i in range(4)] + [int(w[r, 4 * G + g])]
            stream = sum(p << (32 * i) for i, p in enumerate(parts))
            for j in range(GROUP_CODES):
                c = (stream >> (5 * j)) & 31
                t[r, GROUP_W * g + 3 * j:GROUP_W * g + 3 * j + 3] = decode_block(c)
    return t[:, :k]


def gemv_i8(words, s_w, n: int, k: int, x: np.ndarray, s_x=None, y_dtype=np.float16):
    """Batch-1 product y = diag(s_w) T x with int8 x: (acc int32 [n], y).
    Exact: integer products through fp64 BLAS (partial sums below 2^53); the
    epilogue is the int8 one of the 3:4 format, ((fp32(acc) * fp32(s_w)) * s_x)
    rounded to y_dtype."""
    t = unpack(words, n, k).astype(np.float64)
    x = np.asarray(x)
    if x.shape != (k,):
        raise ValueError("x must have shape (k,)")
    acc = (t @ x.astype(np.float64)).astype(np.int64)
    if np.any(np.abs(acc) >= 2 ** 31):
        raise OverflowError("accumulator exceeds int32")
    a = acc.astype(np.float32) * np.asarray(s_w).astype(np.float32)
    if s_x is not None:
        a = a * np.float32(s_x)
    return acc.astype(np.int32), a.astype(y_dtype)
