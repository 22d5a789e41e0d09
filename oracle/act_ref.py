"""Per-token absmax int8 activation quantization: plain CPU reference.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library.

The Sherry paper ("Sherry: Hardware-Efficient 1.25-Bit Ternary Quantization
via Fine-grained Sparsification") quantizes weights; it fixes nothing about
the activations that meet them.  The int8 products take int8 activations
with one scale per token, and the reading taken here is the common symmetric
absmax rule, computed in fp32:
  A1  s = fp32(max_k |x[m, k]|) / 127: one fp32 division, rounded once (RNE);
      a token whose values are all zero takes s = 1;
  A2  x_q = clip(rint(fp32(x) / s), -127, 127): one fp32 division per
      element, rounded once, then rounded to an integer with ties to even;
  A3  fp16 and bf16 inputs are first converted to fp32 (exactly);
      non-finite inputs are a caller error.
Dequantized, x is x_q * s, within s / 2 of fp32(x) (plus the quotient's own
rounding).
"""
from __future__ import annotations

import numpy as np


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values of x given as float32, float16, or bf16 bit patterns
    (uint16): a bf16 pattern is the top half of the fp32 pattern (A3)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32)
    raise ValueError(dtype)


def quantize(x: np.ndarray, dtype: str = "f32"):
    """Rows of x (m x k) -> (x_q int8 [m, k], s fp32 [m]) by A1-A3.

    Token by token: the absmax, one fp32 division for the scale, then one
    fp32 division and a round-half-even per element."""
    xf = to_f32(x, dtype)
    if xf.ndim != 2:
        raise ValueError("x must be m x k")
    m, k = xf.shape
    q = np.zeros((m, k), dtype=np.int8)
    s = np.ones(m, dtype=np.float32)
    for t in range(m):
        row = xf[t]
        amax = np.float32(np.max(np.abs(row))) if k else np.float32(0)
        if amax == 0:
            continue  # s = 1, x_q = 0
        st = np.float32(amax / np.float32(127))  # numpy fp32 / fp32: IEEE division, RNE
        quot = (row / st).astype(np.float32)     # per element, IEEE division
        q[t] = np.clip(np.rint(quot), -127, 127).astype(np.int8)  # rint: ties to even
        s[t] = st
    return q, s
