"""MXFP4 (E2M1 values, one E8M0 scale per 32) for the routed experts — test
infrastructure only.

The model page puts the routed experts in a 4-bit format: E2M1 values with a
scale per small block of inputs, and rounds each expert input to FP4 under
fast-math (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4" and "What
--fast-math does"). Its format uses an E4M3 scale per 16 values; the 4-bit
format that this GPU's block-scaled matrix units take natively is the OCP
microscaling MXFP4: E2M1 elements with one power-of-two (E8M0) scale per 32
consecutive values. This module defines that format, the per-row block
quantisation and the linear layer on it:

* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
  0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6. No infinities or NaN.
* E8M0: an exponent only, value 2**(e - 127) for e in 0..254 (255 is NaN and
  never written).
* Block quantisation (OCP MX v1.0): for a block of 32 values with amax > 0,
  the shared exponent is floor(log2(amax)) - 2 (2 = the exponent of E2M1's
  largest value), clamped to [-127, 127]; each value is divided by the scale
  (exact: a power of two) and rounded to E2M1 to nearest, ties to even, values
  beyond 6 saturating to 6. Readings taken where the standard leaves room: an
  all-zero block gets scale 1 (E8M0 127); the sign of a value that rounds to
  zero is kept (code 0x8).
* Packing: two elements per byte, element 2i in the low nibble of byte i, so
  a row of K values is K/2 bytes and block b of a row is bytes 16b .. 16b + 15.
* Linear: y[m, n] = bf16( sum_b 2**(ea[m,b] + ew[n,b] - 254)
  * sum_{k in block b} dec(a[m, k]) * dec(w[n, k]) ). Every product of two
  E2M1 values is a multiple of 0.25 below 36, so block sums and their
  power-of-two scaling are exact in float64; the float64 sum over blocks is
  exact while the scaled block results span fewer than about 2**40 in
  magnitude, and otherwise off by float64 rounding only.
* Routed experts (``moe_mxfp4_pass``): the chain of the FP8 oracle (routing,
  W13 = [gate; up], h = fl32(silu(g) * u), the router-weighted sum of the
  k copies' outputs at full precision in the order j = 0, 1, ..., rounded
  once to BF16) with every expert input in MXFP4: each
  token's BF16 row quantised once over H, each routed copy's h quantised
  over I. The weights W13[e] [2I, H] and W2[e] [H, I] are MXFP4 along their
  input dimension.
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_to_bf16_bits
from .moe import combine_copies, route, swiglu_f32

__all__ = ["E2M1_MAX", "e2m1_decode", "e2m1_encode", "mx_quantize_rows", "mx_unpack", "mx_dequant",
           "mxfp4_linear", "e8m0_value", "moe_mxfp4_pass", "moe_mxfp4_two_pass"]

E2M1_MAX = 6.0
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64, from the bit fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m * 0.5) * np.exp2(e - 1.0))
    return sign * mag


def e2m1_encode(v) -> np.ndarray:
    """float -> nearest E2M1 code, ties to the even mantissa, |v| > 6 saturating; the sign kept on zero."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    # distance to every magnitude; ties go to the code with mantissa bit 0
    d = np.abs(a[..., None] - _MAG)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    idx = np.arange(8)
    even = (idx & 1) == 0
    pick = np.where(cand & even, idx, 99).min(axis=-1)
    pick = np.where(pick == 99, np.argmax(cand, axis=-1), pick)
    sign = np.signbit(v).astype(np.int64) << 3
    return (pick | sign).astype(np.uint8)


def e8m0_value(e) -> np.ndarray:
    return np.exp2(np.asarray(e, dtype=np.float64) - 127.0)


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exact (from frexp, not a rounded log)."""
    _, ex = np.frexp(a)  # a = f * 2**ex with 0.5 <= f < 1
    return ex.astype(np.int64) - 1


def mx_quantize_rows(x):
    """Rows of float values [M, K] (K a multiple of 32) -> (packed codes uint8
    [M, K/2], E8M0 scales uint8 [M, K/32])."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(M, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    shared = np.zeros_like(amax, dtype=np.int64)
    nz = amax > 0
    shared[nz] = _floor_log2(amax[nz]) - 2
    shared = np.clip(shared, -127, 127)
    scale = np.exp2(shared.astype(np.float64))
    codes = e2m1_encode(blocks / scale[..., None]).reshape(M, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (shared + 127).astype(np.uint8)


def mx_unpack(packed) -> np.ndarray:
    """Packed bytes [M, K/2] -> codes [M, K] (element 2i from the low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def mx_dequant(packed, scales) -> np.ndarray:
    """Packed codes [M, K/2] and E8M0 scales [M, K/32] -> float64 values [M, K] (exact)."""
    vals = e2m1_decode(mx_unpack(packed))
    M, K = vals.shape
    s = e8m0_value(scales)
    return (vals.reshape(M, K // 32, 32) * s[..., None]).reshape(M, K)


def mxfp4_linear(qa, sa, qw, sw):
    """y = bf16(a . w^T) of two MXFP4 operands (rows [M, K] and [N, K]).
    Returns ``(y64, y_bf16)``."""
    y = mx_dequant(qa, sa) @ mx_dequant(qw, sw).T
    return y, round_to_bf16_bits(y)


def moe_mxfp4_pass(x32, ids, w, q13, s13, q2, s2, keep=False):
    """One routed-expert pass with MXFP4 expert inputs and weights.

    ``x32`` float32 [T, H] (BF16 values); ``q13`` [E, 2I, H/2] / ``s13``
    [E, 2I, H/32]; ``q2`` [E, H, I/2] / ``s2`` [E, H, I/32]. Returns
    ``(out64 [T, H], out_bf16 [T, H], extra)``; ``extra`` (with ``keep``)
    holds the token codes and scales, the sorted slots' gate/up values, h, its
    codes and scales, and the permutation.
    """
    x32 = np.asarray(x32, np.float32)
    T = x32.shape[0]
    ids = np.asarray(ids)
    k = ids.shape[1]
    w = np.asarray(w, np.float32).astype(np.float64).reshape(-1)
    E, H = q2.shape[0], q2.shape[1]
    qx, sx = mx_quantize_rows(x32)
    _, offsets, perm = route(ids, E)
    flat_e = ids.reshape(-1)
    gu = np.empty((perm.size, q13.shape[1]), np.float64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if lo == hi:
            continue
        tok = perm[lo:hi] // k
        gu[lo:hi] = mxfp4_linear(qx[tok], sx[tok], q13[e], s13[e])[0]
    h = swiglu_f32(gu)
    qh, sh = mx_quantize_rows(h)
    wy = np.zeros((T * k, H), np.float64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if lo == hi:
            continue
        slots = perm[lo:hi]
        assert np.all(flat_e[slots] == e)
        y = mxfp4_linear(qh[lo:hi], sh[lo:hi], q2[e], s2[e])[0]
        wy[slots] = w[slots][:, None] * y
    out = combine_copies(wy.reshape(T, k, H))
    extra = None
    if keep:
        extra = {"qx": qx, "sx": sx, "gu": gu, "h": h, "qh": qh, "sh": sh, "perm": perm}
    return out, round_to_bf16_bits(out), extra


def moe_mxfp4_two_pass(x32, routes, q13, s13, q2, s2):
    """The stack run twice on one set of MXFP4 expert weights: pass p takes the
    previous pass's BF16 output as its input. Returns [(out64, out_bf16)] per pass."""
    x = np.asarray(x32, np.float32)
    results = []
    for ids, w in routes:
        out64, out_bf16, _ = moe_mxfp4_pass(x, ids, w, q13, s13, q2, s2)
        results.append((out64, out_bf16))
        x = (out_bf16.astype(np.uint32) << 16).view(np.float32)
    return results
