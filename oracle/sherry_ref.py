"""Sherry 3:4 sparse ternary format: plain CPU reference (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library.

What the pages fix ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization
via Fine-grained Sparsification"):
  * Abstract: weights take values in {-1, 0, +1}; a 3:4 fine-grained sparsity
    (one zero in every block of four weights) lets a block of four weights be
    packed into five bits, a regular 1.25-bit width with power-of-two
    alignment.
  * Figure 2 caption: the 4-weight block is the SIMD unit ("4-way patterns"),
    against 2-bit-per-weight packing and 3-weights-in-5-bits packing.

Counting check that makes the format well posed: a block has 4 choices for the
zero slot and 2^3 sign patterns for the other three slots, 4 * 8 = 32 = 2^5, so
block <-> 5-bit code is a bijection and every 5-bit pattern is a valid block.

Readings taken where the pages are silent (each one is listed, with its
justification, in the design notes):
  R1  a block is 4 consecutive weights of one output row along the input
      (reduction) axis: block j of row r is W[r, 4j:4j+4];
  R2  code = z | n0 << 2 | n1 << 3 | n2 << 4, z = zero slot (0..3); n0, n1, n2
      are the sign bits of the three nonzero slots in ascending slot order
      (z skipped); a set sign bit means -1;
  R3  32 codes (128 weights) form a group stored in five little-endian uint32
      words as one LSB-first bitstream: code j occupies bits [5j, 5j + 5) of
      d0 + d1 * 2^32 + ... + d4 * 2^128 (codes 6, 12, 19, 25 straddle words);
  R4  matrix layout row-major, G = K / 128 groups per row, K % 128 == 0; row
      r occupies the 5G words [5Gr, 5G(r+1)): first words 0-3 of every group
      (group g at 5Gr + 4g), then word 4 of every group (group g at
      5Gr + 4G + g).  Each group keeps its five words; splitting them into a
      16-byte part and a 4-byte part lets a GPU read both parts of a row with
      aligned, contiguous loads.  A one-group row is simply its five words;
  R5  packer: zero slot = argmin |w| over the block (lowest slot on ties),
      kept weight negative iff w < 0 (so -0.0 is +1);
  R6  one scale per output row, alpha_r = (sum of kept |w|) / (3K / 4), the
      least-squares scale for the chosen pattern: the sum is exact, the
      division is fp64, and the result is rounded once (RNE) to the scale dtype;
  R7  int8 epilogue y = dtype( (fp32(acc) * fp32(s_w[r])) * s_x ), left to
      right in fp32 with round-to-nearest-even and no fused multiply-add.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 4
GROUP_BLOCKS = 32
GROUP_WEIGHTS = BLOCK * GROUP_BLOCKS  # 128
GROUP_WORDS = 5  # 32 codes * 5 bits = 160 bits = 5 uint32
N_CODES = 32


def check_shape(n: int, k: int) -> None:
    if n <= 0 or k <= 0:
        raise ValueError(f"n and k must be positive, got n={n} k={k}")
    if k % GROUP_WEIGHTS:
        raise ValueError(f"k={k} must be a multiple of {GROUP_WEIGHTS} (no code means an all-zero block)")


def packed_bytes(n: int, k: int) -> int:
    """Bytes of the code payload: 5 bits per 4 weights, n*k*5/32 (1.25 b/w)."""
    check_shape(n, k)
    return n * (k // GROUP_WEIGHTS) * GROUP_WORDS * 4


# --------------------------------------------------------------------------
# One block (pure Python, readings R2 and R5)
# --------------------------------------------------------------------------

def decode_block(c: int) -> tuple:
    """5-bit code -> the four ternary weights of its block (R2)."""
    c = int(c)
    if not 0 <= c < N_CODES:
        raise ValueError(f"code {c} outside [0, 32)")
    z = c & 3
    sign_bits = c >> 2
    out = []
    k = 0
    for slot in range(BLOCK):
        if slot == z:
            out.append(0)
        else:
            out.append(-1 if (sign_bits >> k) & 1 else 1)
            k += 1
    return tuple(out)


def encode_block(t) -> int:
    """Four ternary weights with exactly one zero -> 5-bit code (inverse of R2)."""
    t = tuple(int(v) for v in t)
    if len(t) != BLOCK or any(v not in (-1, 0, 1) for v in t):
        raise ValueError(f"not a ternary block of 4: {t}")
    if t.count(0) != 1:
        raise ValueError(f"3:4 block needs exactly one zero: {t}")
    z = t.index(0)
    code = z
    k = 0
    for slot in range(BLOCK):
        if slot == z:
            continue
        if t[slot] < 0:
            code |= 1 << (2 + k)
        k += 1
    return code


def quantize_block(w4) -> int:
    """Real block -> code: zero the smallest |w| (lowest slot on ties), keep
    the signs of the other three (R5)."""
    w4 = [float(v) for v in w4]
    if len(w4) != BLOCK or not all(math.isfinite(v) for v in w4):
        raise ValueError("need 4 finite weights")
    z = min(range(BLOCK), key=lambda s: (abs(w4[s]), s))
    t = [0] * BLOCK
    for slot in range(BLOCK):
        if slot != z:
            t[slot] = -1 if w4[slot] < 0 else 1
    return encode_block(t)


# --------------------------------------------------------------------------
# One group of 32 codes <-> 5 words (pure Python, reading R3)
# --------------------------------------------------------------------------

def pack_group(codes32) -> list:
    codes32 = [int(c) for c in codes32]
    if len(codes32) != GROUP_BLOCKS or any(not 0 <= c < N_CODES for c in codes32):
        raise ValueError("need 32 codes in [0, 32)")
    v = 0
    for j, c in enumerate(codes32):
        v |= c << (5 * j)
    return [(v >> (32 * i)) & 0xFFFFFFFF for i in range(GROUP_WORDS)]


def unpack_group(words5) -> list:
    words5 = [int(w) for w in words5]
    if len(words5) != GROUP_WORDS:
        raise ValueError("need 5 words")
    v = 0
    for i, w in enumerate(words5):
        v |= (w & 0xFFFFFFFF) << (32 * i)
    return [(v >> (5 * j)) & 31 for j in range(GROUP_BLOCKS)]


# --------------------------------------------------------------------------
# Whole matrices (numpy, same readings, vectorised)
# --------------------------------------------------------------------------

def codes_from_dense(t: np.ndarray) -> np.ndarray:
    """int8 [n, k] 3:4 ternary -> uint8 codes [n, k/4] (raises if any block is
    not exactly one zero plus three +-1)."""
    t = np.asarray(t)
    n, k = t.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 4")
    b = t.reshape(n, k // BLOCK, BLOCK).astype(np.int64)
    if np.any((b != -1) & (b != 0) & (b != 1)):
        raise ValueError("entries must be -1, 0 or +1")
    zeros = b == 0
    if np.any(zeros.sum(axis=2) != 1):
        raise ValueError("every block of 4 must hold exactly one zero")
    z = np.argmax(zeros, axis=2)
    code = z.copy()
    k_idx = np.zeros_like(z)
    for slot in range(BLOCK):
        is_nz = slot != z
        neg = is_nz & (b[:, :, slot] < 0)
        code |= np.where(neg, 1 << (2 + k_idx), 0)
        k_idx = k_idx + is_nz
    return code.astype(np.uint8)


def dense_from_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [n, k/4] -> int8 [n, k] ternary (R2)."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c >= N_CODES)):
        raise ValueError("codes must be in [0, 32)")
    n, nb = c.shape
    z = c & 3
    s = c >> 2
    out = np.zeros((n, nb, BLOCK), dtype=np.int8)
    for slot in range(BLOCK):
        k_idx = slot - (slot > z)  # position among the nonzero slots
        bit = (s >> k_idx) & 1
        out[:, :, slot] = np.where(slot == z, 0, 1 - 2 * bit)
    return out.reshape(n, nb * BLOCK)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [n, k/4] -> uint32 words [n * G * 5] (R3, R4): each group's
    160 bits as an LSB-first stream, 5 bits per code, giving words d0..d4;
    per row the d0..d3 of every group come first, then the d4 of every group."""
    c = np.asarray(codes).astype(np.uint8)
    n, nb = c.shape
    if nb % GROUP_BLOCKS:
        raise ValueError("k/4 must be a multiple of 32")
    if np.any(c >= N_CODES):
        raise ValueError("codes must be in [0, 32)")
    g = nb // GROUP_BLOCKS
    bits = np.unpackbits(c[:, :, None], axis=2, bitorder="little")[:, :, :5]  # [n, nb, 5]
    bits = bits.reshape(n, g, GROUP_BLOCKS * 5)  # 160 bits per group
    by = np.packbits(bits, axis=2, bitorder="little")  # [n, G, 20] bytes
    d = np.ascontiguousarray(by).reshape(-1).view("<u4").astype(np.uint32).reshape(n, g, GROUP_WORDS)
    return np.concatenate([d[:, :, :4].reshape(n, 4 * g), d[:, :, 4]], axis=1).reshape(-1)


def group_words(words: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed words (layout R4) -> uint32 [n, G, 5]: d0..d4 of every group."""
    check_shape(n, k)
    g = k // GROUP_WEIGHTS
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    if w.size != n * g * GROUP_WORDS:
        raise ValueError(f"expected {n * g * GROUP_WORDS} words, got {w.size}")
    w = w.reshape(n, GROUP_WORDS * g)
    out = np.empty((n, g, GROUP_WORDS), dtype=np.uint32)
    out[:, :, :4] = w[:, :4 * g].reshape(n, g, 4)
    out[:, :, 4] = w[:, 4 * g:]
    return out


def unpack_codes(words: np.ndarray, n: int, k: int) -> np.ndarray:
    """uint32 words [n * G * 5] -> uint8 codes [n, k/4] (inverse of pack_codes)."""
    d = group_words(words, n, k)
    g = d.shape[1]
    by = np.ascontiguousarray(d).astype("<u4").view(np.uint8).reshape(n, g, GROUP_WORDS * 4)
    bits = np.unpackbits(by, axis=2, bitorder="little").reshape(n, g, GROUP_BLOCKS, 5)
    weights = (1 << np.arange(5)).astype(np.uint8)
    codes = (bits * weights).sum(axis=3).astype(np.uint8)
    return codes.reshape(n, g * GROUP_BLOCKS)


def row_words(words: np.ndarray, n: int, k: int, rows) -> np.ndarray:
    """The words of the given rows, in order (rows are contiguous in R4)."""
    check_shape(n, k)
    per = (k // GROUP_WEIGHTS) * GROUP_WORDS
    w = np.asarray(words, dtype=np.uint32).reshape(n, per)
    return np.ascontiguousarray(w[np.asarray(rows)]).reshape(-1)


def unpack(words: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed words -> dense int8 ternary matrix [n, k]."""
    return dense_from_codes(unpack_codes(words, n, k))


def quantize(w: np.ndarray):
    """Real matrix [n, k] -> (codes uint8 [n, k/4], alpha fp64 [n]) by R5/R6.

    alpha_r is the exact sum of the kept magnitudes (math.fsum over the exact
    fp64 images of the inputs) divided in fp64 by the kept count 3k/4."""
    w = np.asarray(w)
    n, k = w.shape
    check_shape(n, k)
    w64 = w.astype(np.float64)
    if not np.all(np.isfinite(w64)):
        raise ValueError("weights must be finite")
    b = w64.reshape(n, k // BLOCK, BLOCK)
    mag = np.abs(b)
    z = np.argmin(mag, axis=2)  # first minimum = lowest slot on ties
    slot = np.arange(BLOCK)[None, None, :]
    kept = slot != z[:, :, None]
    t = np.where(kept, np.where(b < 0, -1, 1), 0).astype(np.int8).reshape(n, k)
    codes = codes_from_dense(t)
    kept_count = 3 * k // 4
    alpha = np.empty(n, dtype=np.float64)
    kept_mag = np.where(kept, mag, 0.0).reshape(n, k)
    for r in range(n):
        alpha[r] = math.fsum(kept_mag[r].tolist()) / kept_count
    return codes, alpha


def pack(w: np.ndarray, scale_dtype=np.float16):
    """Real matrix -> (packed words uint32 [n*G*5], per-row scales)."""
    codes, alpha = quantize(w)
    return pack_codes(codes), alpha.astype(scale_dtype)


# --------------------------------------------------------------------------
# Products
# --------------------------------------------------------------------------

def _exact_int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Integer product via fp64 BLAS.  Exact here: every operand is an integer
    of magnitude <= 127 and every partial sum is bounded by 127 * k < 2^53."""
    k = a.shape[-1]
    if 127 * 127 * k >= 2 ** 53:
        raise ValueError("k too large for an exact fp64 integer product")
    r = a.astype(np.float64) @ b.astype(np.float64)
    out = r.astype(np.int64)
    if np.any(np.abs(out) >= 2 ** 31):
        raise OverflowError("accumulator exceeds int32")
    return out


def epilogue(acc: np.ndarray, s_w: np.ndarray, s_x=None, y_dtype=np.float16) -> np.ndarray:
    """R7: y = y_dtype((fp32(acc) * fp32(s_w)) * s_x), numpy float32 IEEE RNE.
    acc is [n] or [m, n]; s_x is None (1.0), a scalar, or [m] per token."""
    a = np.asarray(acc).astype(np.float32)  # exact: |acc| < 2^24
    t = a * np.asarray(s_w).astype(np.float32)
    if s_x is not None:
        sx = np.asarray(s_x, dtype=np.float32)
        t = t * (sx[:, None] if sx.ndim == 1 and t.ndim == 2 else sx)
    return t.astype(y_dtype)


def gemv_i8(words, s_w, n: int, k: int, x: np.ndarray, s_x=None, y_dtype=np.float16):
    """Batch-1 product y = diag(s_w) T x with int8 x: returns (acc int32 [n], y)."""
    t = unpack(words, n, k)
    x = np.asarray(x)
    if x.shape != (k,):
        raise ValueError("x must have shape (k,)")
    acc = _exact_int_matmul(t, x.astype(np.int64)).astype(np.int32)
    return acc, epilogue(acc, s_w, s_x, y_dtype)


def gemm_i8(words, s_w, n: int, k: int, x: np.ndarray, s_x, y_dtype=np.float16):
    """Y[m, n] = s_x[m] * s_w[n] * sum_k X[m, k] T[n, k]; returns (acc int32
    [m, n], y [m, n]).  Per element the epilogue is (acc * s_w[n]) * s_x[m]."""
    t = unpack(words, n, k)
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] != k:
        raise ValueError("x must be [m, k]")
    acc = _exact_int_matmul(x.astype(np.int64), t.T.astype(np.int64)).astype(np.int32)
    return acc, epilogue(acc, s_w, s_x, y_dtype)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _exact_rows_dot(t: np.ndarray, x64: np.ndarray) -> np.ndarray:
    """sum_k t[r, k] * x[k] exactly, rounded once to fp64.  Uses fp64 BLAS when
    every partial sum is a multiple of the smallest ulp in x and below 2^53 of
    them (then BLAS is exact), else math.fsum row by row."""
    nz = x64[x64 != 0]
    if nz.size == 0:
        return np.zeros(t.shape[0])
    e_min = np.min(np.frexp(nz)[1]) - 8  # bf16: 8 significant bits
    bound = float(np.sum(np.abs(x64)))
    if bound * 2.0 ** (-e_min) < 2.0 ** 52:
        return t.astype(np.float64) @ x64
    return np.array([math.fsum((t[r] * x64).tolist()) for r in range(t.shape[0])])


def gemv_bf16(words, s_w, n: int, k: int, x_bits: np.ndarray) -> np.ndarray:
    """Batch-1 product with bf16 x: the exact value s_w[r] * sum_k T[r, k] x[k]
    in fp64 (one rounding for the sum, one for the scale product)."""
    t = unpack(words, n, k)
    x64 = bf16_bits_to_f64(x_bits)
    if x64.shape != (k,):
        raise ValueError("x must have shape (k,)")
    return _exact_rows_dot(t, x64) * np.asarray(s_w).astype(np.float64)


def gemm_bf16(words, s_w, n: int, k: int, x_bits: np.ndarray) -> np.ndarray:
    """Product for M tokens with bf16 X [m, k]: Y[m, r] = s_w[r] * sum_k
    T[r, k] X[m, k], each token's sums exact and rounded once to fp64, then
    one rounding for the scale product (the batch-1 rule, token by token).
    Returns fp64 [m, n]."""
    t = unpack(words, n, k)
    xb = np.asarray(x_bits)
    if xb.ndim != 2 or xb.shape[1] != k:
        raise ValueError("x must be [m, k]")
    sw = np.asarray(s_w).astype(np.float64)
    return np.stack([_exact_rows_dot(t, bf16_bits_to_f64(xb[i])) * sw for i in range(xb.shape[0])])
