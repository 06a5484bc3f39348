"""The W8A8 linear layer of the oracle — test infrastructure only.

What the layer computes (Lernex/Metis-1.6-Logos-FP8, "What --fast-math
does"): the input is converted to FP8 with a scale per token and the
product with the FP8 weights is formed. The same page's "Benchmarks"
section evaluates the FP8 model by decoding the stored weights exactly and
feeding every quantised layer a per-token FP8 version of its input; that
emulation is this oracle:

    Y[m, n] = bf16( s_x[m] * s_w[n] * sum_k dec(qx[m, k]) * dec(qw[n, k]) )

with the weights stored [out, in] and one scale per output row (Lernex/
Metis-1.6-Praxis-NVFP4, "What is in NVFP4"). There is no bias.

Exactness: every decoded E4M3 value times 2**9 is an integer of magnitude
at most 448 * 2**9 < 2**18, so each product is an integer multiple of
2**-18 below 2**36 units, and any partial sum over K < 2**17 terms stays
below 2**53 units. The float64 matrix product is therefore exact in any
summation order; ``w8a8_linear_int`` computes the same sums on int64 and
is used to confirm that. The product of the two float32 scales is exact in
float64, so the only roundings are one float64 rounding of the scaled sum
and the final BF16 rounding.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16_bits
from .e4m3 import decode

__all__ = ["w8a8_linear", "w8a8_linear_int", "dequant_sum", "w8a16_linear"]


def dequant_sum(qa, qb) -> np.ndarray:
    """acc[m, n] = sum_k dec(qa[m, k]) * dec(qb[n, k]) in float64 (exact)."""
    a = decode(qa)
    b = decode(qb)
    return a @ b.T


def w8a8_linear(qx, sx, qw, sw):
    """Return ``(y64 float64 [M,N], y_bf16 uint16 [M,N])``."""
    qx = np.asarray(qx, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    acc = dequant_sum(qx, qw)
    scale = np.asarray(sx, np.float32).astype(np.float64)[:, None] * \
        np.asarray(sw, np.float32).astype(np.float64)[None, :]
    y = scale * acc
    return y, round_to_bf16_bits(y)


def _code_to_int512(codes) -> np.ndarray:
    """Integer value of dec(code) * 2**9, computed from the bit fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1, 1)
    e = (c >> 3) & 0xF
    m = c & 7
    # normal: (8 + m) * 2**(e - 7 - 3) * 2**9 = (8 + m) << (e - 1); subnormal: m * 2**-9 * 2**9 = m
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return sign * mag


def w8a8_linear_int(qx, qw) -> np.ndarray:
    """The same sums as ``dequant_sum`` on int64, in units of 2**-18.

    NaN codes are not representable here; callers pass finite codes only.
    """
    a = _code_to_int512(qx)
    b = _code_to_int512(qw)
    return a @ b.T


def w8a16_linear(x_bits, qw, sw):
    """The default maths: BF16 activations times the exactly decoded weights.

    Lernex/Metis-1.6-Logos-FP8, "What --fast-math does": without the flag the
    FP8 weights are widened to 16 bits and the product is taken in BF16, so
    only the weights are rounded (the activations are not quantised):

        Y[m, n] = bf16( s_w[n] * sum_k x[m, k] * dec(qw[n, k]) )

    ``x_bits`` are BF16 bit patterns [M, K]. Returns ``(y64, y_bf16)``.

    Precision: each product of a BF16 value (8 significant bits) and an E4M3
    value (4) is exact in float64; the float64 sum differs from the exact one
    by at most K * 2**-53 * sum |x w|, far below the BF16 output rounding.
    """
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    w = decode(np.asarray(qw, dtype=np.uint8))
    y = (x @ w.T) * np.asarray(sw, np.float32).astype(np.float64)[None, :]
    return y, round_to_bf16_bits(y)
