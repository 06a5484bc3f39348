"""BF16 rounding of the oracle — test infrastructure only.

The layer's output is BF16, the model's own dtype (Lernex/Metis-1.6-Logos-
FP8, "What --fast-math does": the default maths runs in BF16). The oracle
rounds a float64 result to BF16 once, to nearest with ties to even, with
BF16's own subnormals (quantum 2**-133) and overflow to infinity; there is
no intermediate float32 step.
"""
from __future__ import annotations

import numpy as np

__all__ = ["round_to_bf16_bits", "bf16_bits_to_f64"]

_BF16_SIG_BITS = 8            # significand bits including the implicit one
_BF16_MIN_QUANTUM_EXP = -133  # subnormal spacing 2**-133


def round_to_bf16_bits(y) -> np.ndarray:
    """float64 -> BF16 bit patterns (uint16), one round-half-to-even step."""
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    finite = np.isfinite(y)
    yf = np.where(finite, y, 0.0)
    _, e = np.frexp(yf)                       # |y| in [2**(e-1), 2**e)
    q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_QUANTUM_EXP)
    r = np.rint(np.ldexp(yf, -q))             # exact scaling, then half-to-even
    val = np.ldexp(r, q)                      # exactly representable in BF16 or >= 2**128
    with np.errstate(over="ignore"):
        f32 = val.astype(np.float32)          # exact, or +-inf past the BF16 range
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    # keep the sign of a zero result (e.g. -1e-300 -> -0)
    bits = np.where((r == 0) & np.signbit(yf), np.uint16(0x8000), bits)
    out[...] = bits
    if not finite.all():
        nf = ~finite
        f = y[nf].astype(np.float32)
        out[nf] = (f.view(np.uint32) >> 16).astype(np.uint16) | np.where(np.isnan(f), 0x40, 0).astype(np.uint16)
    return out


def bf16_bits_to_f64(b) -> np.ndarray:
    """BF16 bit patterns -> float64, exact."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
