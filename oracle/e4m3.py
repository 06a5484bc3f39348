"""E4M3 (FP8) codec of the oracle — test infrastructure only.

The pages store weights as FP8 E4M3 (Lernex/Metis-1.6-Logos-FP8, "What is
in FP8") with safetensors tensor type F8_E4M3 (Lernex/Metis-1.6-Praxis-
NVFP4, hub sidebar). They do not print the bit layout; the reading taken
here is the OCP 8-bit "E4M3FN" format that tensor type names: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN only at
S.1111.111, largest finite magnitude 448, smallest subnormal 2**-9.

Encoding is round to nearest, ties to the even code, with saturation:
magnitudes at or above 448 become 448. The sign of the input is kept, so a
negative value that rounds to zero gives the code 0x80.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0

__all__ = ["E4M3_MAX", "decode_table", "decode", "magnitudes", "finite_codes", "encode",
           "encode_bits"]


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6          # subnormal
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)  # normal


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
_TABLE.setflags(write=False)


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN at 0x7F and 0xFF)."""
    return _TABLE


def decode(codes) -> np.ndarray:
    """Exact float64 values of an array of uint8 codes."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def finite_codes() -> np.ndarray:
    """The 254 codes with a finite value (both zeros included)."""
    c = np.arange(256, dtype=np.uint8)
    return c[~np.isnan(_TABLE)]


# Codes 0x00..0x7E hold the 127 non-negative magnitudes in increasing order.
_MAG = _TABLE[:127].copy()
_MAG.setflags(write=False)
assert np.all(np.diff(_MAG) > 0)


def magnitudes() -> np.ndarray:
    """The 127 representable magnitudes, ascending; index == code."""
    return _MAG


def encode(v) -> np.ndarray:
    """float32 values -> E4M3 codes: nearest magnitude, ties to even, saturating.

    Written as a search over the table of magnitudes: the code whose value is
    closest to |v| wins; on an exact tie the code with mantissa bit 0 (an
    even code, since magnitude codes are consecutive integers) wins. |v| at
    or above 448 saturates to 448. NaN gives 0x7F.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(_MAG, a, side="left")          # first magnitude >= a
    hi = np.clip(hi, 1, 126)
    lo = hi - 1
    d_lo = a - _MAG[lo]
    d_hi = _MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= E4M3_MAX, 126, mag)
    code = mag.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def encode_bits(v) -> np.ndarray:
    """Second, independent encoder written on the float32 bit fields.

    Used only to cross-check ``encode``. For a normal E4M3 result the top
    three fraction bits of the float32 are kept and the remaining twenty
    decide the rounding (round half to even); below 2**-6 the value is an
    integer multiple of 2**-9 and is rounded as such.
    """
    v = np.asarray(v, dtype=np.float32)
    bits = v.view(np.uint32).astype(np.int64)
    sign = (bits >> 31) & 1
    a = bits & 0x7FFFFFFF
    exp32 = a >> 23
    frac = a & 0x7FFFFF
    # normal range: 2**-6 <= |v|, exponent field of the result = exp32 - 127 + 7
    e8 = exp32 - 120
    top = frac >> 20
    rest = frac & 0xFFFFF
    code_n = (e8 << 3) | top
    up = (rest > 0x80000) | ((rest == 0x80000) & ((code_n & 1) == 1))
    code_n = code_n + up.astype(np.int64)
    # subnormal range: |v| < 2**-6 -> multiple of 2**-9, computed on integers
    # value = (2**23 + frac) * 2**(exp32 - 150) for normal float32, frac * 2**-149 otherwise
    sig = np.where(exp32 > 0, frac | (1 << 23), frac)
    e_eff = np.where(exp32 > 0, exp32, 1)
    # |v| / 2**-9 = sig * 2**(e_eff - 150 + 9) = sig / 2**(141 - e_eff)
    shift = 141 - e_eff                                # >= 141-120 = 21 in this range
    shift_c = np.clip(shift, 0, 62)
    q = sig >> shift_c
    rem = sig - (q << shift_c)
    half = np.where(shift_c > 0, np.int64(1) << np.maximum(shift_c - 1, 0), 0)
    up_s = (rem > half) | ((rem == half) & ((q & 1) == 1))
    code_s = np.where(shift > 62, 0, q + up_s.astype(np.int64))
    code = np.where(a >= 0x3C800000, code_n, code_s)
    code = np.where(a >= 0x43E00000, 126, code)        # |v| >= 448 saturates
    out = (code | (sign << 7)).astype(np.uint8)
    return np.where(a > 0x7F800000, np.uint8(0x7F), out).astype(np.uint8)
