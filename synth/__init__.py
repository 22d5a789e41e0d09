"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only draws random inputs with the shapes and distributions of the
workloads; it holds none of the format's arithmetic (no encoding, decoding,
packing or products).  Everything is driven by ``numpy.random.Generator``
(PCG64) seeds so both sides see the same bytes.

Workloads (shapes from the LLaMA-3.2 models the Sherry paper evaluates,
"Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization via Fine-grained
Sparsification", Abstract):
  * single matrix 256x1024, int8 x uniform in [-127, 127], fp32 row scales;
  * LLaMA-3.2-1B decoder layer (q, k, v, o, gate, up, down), batch 1;
  * LLaMA-3.2-3B decoder layer, bf16 activations;
  * 1B layer at M in {2, 4, 8, 16} tokens and at M = 2048 (prefill).
"""
from __future__ import annotations

import numpy as np

# (name, n_out, k_in) for one decoder layer.
LLAMA32_1B_LAYER = (
    ("q", 2048, 2048),
    ("k", 512, 2048),
    ("v", 512, 2048),
    ("o", 2048, 2048),
    ("gate", 8192, 2048),
    ("up", 8192, 2048),
    ("down", 2048, 8192),
)
LLAMA32_3B_LAYER = (
    ("q", 3072, 3072),
    ("k", 1024, 3072),
    ("v", 1024, 3072),
    ("o", 3072, 3072),
    ("gate", 8192, 3072),
    ("up", 8192, 3072),
    ("down", 3072, 8192),
)
SINGLE_MATRIX = (("w", 256, 1024),)
SMALL_BATCH_M = (2, 4, 8, 16)
PREFILL_M = 2048


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.PCG64(seed))


def ternary_34(n: int, k: int, g: np.random.Generator) -> np.ndarray:
    """Dense int8 [n, k] ternary matrix with exactly one zero in every run of 4
    consecutive entries along k: zero position uniform over the 4 slots, the
    other three entries +1/-1 by a fair coin.  k must be a multiple of 4."""
    if k % 4:
        raise ValueError("k must be a multiple of 4")
    nb = k // 4
    zpos = g.integers(0, 4, size=(n, nb))
    signs = g.integers(0, 2, size=(n, nb, 4)).astype(np.int8) * 2 - 1
    t = signs.copy()
    t[np.arange(n)[:, None], np.arange(nb)[None, :], zpos] = 0
    return t.reshape(n, k).astype(np.int8)


def ternary_dense(n: int, k: int, g: np.random.Generator, p_zero: float = 1.0 / 3.0) -> np.ndarray:
    """Dense int8 ternary matrix with no block structure (i.i.d. entries)."""
    u = g.random((n, k))
    t = np.where(u < p_zero, 0, np.where(g.random((n, k)) < 0.5, -1, 1))
    return t.astype(np.int8)


def random_words(n_words: int, g: np.random.Generator) -> np.ndarray:
    """Uniform random 32-bit words.  Every 5-bit pattern is a valid block code,
    so uniform random packed words are uniform random 3:4 ternary matrices."""
    return g.integers(0, 1 << 32, size=n_words, dtype=np.uint64).astype(np.uint32)


def row_scales(n: int, g: np.random.Generator, dtype=np.float16, lo=0.01, hi=0.1) -> np.ndarray:
    """Per-row scales drawn U[lo, hi] in fp64 then rounded (RNE) to dtype."""
    return g.uniform(lo, hi, size=n).astype(dtype)


def x_int8_uniform(shape, g: np.random.Generator) -> np.ndarray:
    return g.integers(-127, 128, size=shape).astype(np.int8)


def act_absmax_int8(m: int, k: int, g: np.random.Generator):
    """Per-token absmax int8 activations from N(0, 1) floats.

    s = fp32(max|x|) / 127 in fp32, x_q = clip(rint(fp32(x) / s), -127, 127)
    with round-half-even; an all-zero token gets s = 1.  Returns (x_q int8
    [m, k], s fp32 [m], x fp32 [m, k])."""
    x = g.standard_normal((m, k)).astype(np.float32)
    amax = np.max(np.abs(x), axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = np.rint(x / s[:, None]).astype(np.float32)
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s, x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest even) and return the 16-bit
    patterns as uint16.  Inputs here are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def x_bf16_normal(shape, g: np.random.Generator) -> np.ndarray:
    """bf16 bit patterns of N(0, 1) draws (RNE from fp32)."""
    return f32_to_bf16_bits(g.standard_normal(shape).astype(np.float32))


def matrix_seed(config_seed: int, index: int) -> int:
    return config_seed * 100 + index
