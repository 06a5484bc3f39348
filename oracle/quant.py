"""Per-row dynamic FP8 quantisation of the oracle — test infrastructure only.

The scheme (Lernex/Metis-1.6-Logos-FP8, "What is in FP8"; sglang-metis
0.1.0, "Serve", memory paragraph): activations are quantised per token at
run time, weights carry one scale per output channel, i.e. per row of the
[out, in] matrix (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4": one
scale per output row). Both are the same map applied to a row.

The pages fix neither the scale formula nor the arithmetic. The readings
taken here, for one row x of float32 values:

* amax = max |x_k| (exact);
* the scale is s = fl32(amax / 448), so the largest element lands on the
  largest E4M3 magnitude; an all-zero row gets s = 1;
* each element is divided by the scale in float32, v_k = fl32(x_k / s), a
  correctly rounded division, and v_k is encoded to E4M3 by round to
  nearest even with saturation at 448 (``oracle.e4m3.encode``);
* float32 subnormals are kept (no flush to zero).

fl32 of a quotient of two float32 numbers is obtained as the float32
rounding of the float64 quotient; rounding twice is harmless for division
because 53 >= 2*24 + 2.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, encode

__all__ = ["bf16_bits_to_f32", "quantize_rows", "row_scale"]


def bf16_bits_to_f32(b) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32, exact."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def row_scale(amax) -> np.ndarray:
    """s = fl32(amax / 448), with s = 1 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax.astype(np.float64) / E4M3_MAX).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_rows(x):
    """Quantise each row of a float32 matrix to E4M3 with one float32 scale.

    Returns ``(q uint8 [M,K], s float32 [M], v float32 [M,K])`` where v is
    the scaled value fed to the encoder (kept for diagnostics).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    if x.shape[1] == 0:
        return (np.zeros(x.shape, np.uint8), np.ones(x.shape[0], np.float32),
                np.zeros(x.shape, np.float32))
    amax = np.max(np.abs(x), axis=1)
    s = row_scale(amax)
    v = (x.astype(np.float64) / s.astype(np.float64)[:, None]).astype(np.float32)
    q = encode(v)
    return q, s, v
