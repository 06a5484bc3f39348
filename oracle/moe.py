"""The routed-expert chain of the oracle — test infrastructure only.

The pages put the routed experts in FP8 with the same scheme as the other
large matrices (Lernex/Metis-1.6-Logos-FP8, "What is in FP8"), route each
token to its top-k experts (Lernex/Metis-1.6-Praxis, "Architecture": four
routed experts per token; Lernex/Metis-1.6-Logos, "Architecture"), store the
experts in global expert order (the "Files" section of both model pages),
and run the whole stack twice per token with one set of weights (sglang-
metis 0.1.0, "How the model maps onto SGLang"; Lernex/Metis-1.6-Praxis,
"Architecture").

The pages leave open the expert's activation, how the gate and up halves
are laid out, how the expert input is requantised and how the k outputs are
combined. Readings taken (each also listed with the other readings in the
design notes):

* W13[e] is [2I, H]; rows 0..I-1 are the gate, rows I..2I-1 the up
  projection; the activation is SwiGLU, h = silu(g) * u with
  silu(g) = g / (1 + exp(-g)).
* Each token is quantised once over H; its k routed copies share that
  scale. h is rounded to float32 (not BF16) and requantised per routed
  copy (slot) with the same per-row quantiser.
* The down projection W2[e] is [H, I]. A token's output is the router-
  weighted sum of its k routed copies' outputs, taken at full precision and
  rounded once to BF16 (the model's dtype): out[t] = bf16(sum_j w[t,j] *
  y[t,j]). No page puts a rounding between the expert stage and that sum,
  so none is placed there. The copies are added in the fixed order
  j = 0, 1, ..., k-1, which makes the float64 sum independent of expert
  labels and of the sorted order. Router weights are inputs and are not
  renormalised here.
* Slots are the flat indices t*k + j. The expert-sorted order is a stable
  sort of the slots by expert id; ids outside [0, E) are dropped and
  contribute nothing.
"""
from __future__ import annotations

import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16_bits
from .linear import dequant_sum
from .quant import quantize_rows

__all__ = ["route", "grouped_gate_up", "swiglu_f32", "bf16_values", "combine_copies", "moe_pass",
           "moe_two_pass"]


def route(ids, E: int):
    """Expert-sorted order of the routed slots.

    Returns ``(counts int64 [E], offsets int64 [E+1], perm int64 [n_valid])``
    where ``perm[offsets[e]:offsets[e+1]]`` lists, in increasing order, the
    flat slot indices t*k + j whose id is e.
    """
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)
    perm = np.argsort(key, kind="stable")[: int(valid.sum())]
    counts = np.bincount(flat[valid], minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return counts, offsets, perm


def grouped_gate_up(qx, sx, ids, qw13, s13):
    """Gate/up products of every routed slot, in expert-sorted order.

    ``gu[r] = s_x[t] * s13[e] * (dec(qx[t]) . dec(W13[e])^T)`` for the r-th
    sorted slot (t, e). Returns ``(gu64 float64 [n_valid, 2I], perm)``.
    """
    qx = np.asarray(qx, np.uint8)
    sx = np.asarray(sx, np.float32).astype(np.float64)
    ids = np.asarray(ids)
    E = qw13.shape[0]
    k = ids.shape[1]
    counts, offsets, perm = route(ids, E)
    gu = np.empty((perm.size, qw13.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if lo == hi:
            continue
        tok = perm[lo:hi] // k
        acc = dequant_sum(qx[tok], qw13[e])
        scale = sx[tok][:, None] * np.asarray(s13[e], np.float32).astype(np.float64)[None, :]
        gu[lo:hi] = scale * acc
    return gu, perm


def swiglu_f32(gu) -> np.ndarray:
    """h = fl32(silu(g) * u) from float64 gate/up rows [n, 2I] -> float32 [n, I]."""
    gu = np.asarray(gu, dtype=np.float64)
    I = gu.shape[1] // 2
    g = gu[:, :I]
    u = gu[:, I:]
    return (g / (1.0 + np.exp(-g)) * u).astype(np.float32)


def bf16_values(y) -> np.ndarray:
    """float64 -> the float64 value of its nearest-even BF16."""
    return bf16_bits_to_f64(round_to_bf16_bits(y))


def combine_copies(wy) -> np.ndarray:
    """sum_j wy[:, j, :] over the top-k positions in the order j = 0, 1, ...
    (float64; a dropped slot's row is zero)."""
    wy = np.asarray(wy, dtype=np.float64)
    out = wy[:, 0, :].copy()
    for j in range(1, wy.shape[1]):
        out += wy[:, j, :]
    return out


def moe_pass(qx, sx, ids, w, qw13, s13, qw2, s2, keep=False):
    """One routed-expert pass on quantised tokens.

    Returns ``(out64 float64 [T,H], out_bf16 uint16 [T,H], extra)`` where
    ``extra`` (only when ``keep``) holds the sorted slots' gate/up values,
    h, its requantised bytes and scales, and the permutation.
    """
    qx = np.asarray(qx, np.uint8)
    T = qx.shape[0]
    ids = np.asarray(ids)
    k = ids.shape[1]
    w = np.asarray(w, np.float32).astype(np.float64).reshape(-1)
    E, H = qw2.shape[0], qw2.shape[1]
    gu, perm = grouped_gate_up(qx, sx, ids, qw13, s13)
    h = swiglu_f32(gu)
    qh, sh, vh = quantize_rows(h)
    _, offsets, _ = route(ids, E)
    flat_e = np.asarray(ids).reshape(-1)
    # the weighted product of every routed copy, in float64, on its slot's row
    wy = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if lo == hi:
            continue
        slots = perm[lo:hi]
        assert np.all(flat_e[slots] == e)
        acc = dequant_sum(qh[lo:hi], qw2[e])
        y = (sh[lo:hi].astype(np.float64)[:, None] *
             np.asarray(s2[e], np.float32).astype(np.float64)[None, :]) * acc
        wy[slots] = w[slots][:, None] * y
    out = combine_copies(wy.reshape(T, k, H))
    extra = None
    if keep:
        extra = {"gu": gu, "h": h, "qh": qh, "sh": sh, "vh": vh, "perm": perm}
    return out, round_to_bf16_bits(out), extra


def moe_two_pass(x_bf16_f32, routes, qw13, s13, qw2, s2):
    """The stack run twice with the same expert weights.

    Pass p quantises its BF16 input per token, runs ``moe_pass`` with that
    pass's routing, and hands its BF16 output to the next pass. Returns the
    list of per-pass ``(out64, out_bf16)``.
    """
    x = np.asarray(x_bf16_f32, dtype=np.float32)
    results = []
    for ids, w in routes:
        qx, sx, _ = quantize_rows(x)
        out64, out_bf16, _ = moe_pass(qx, sx, ids, w, qw13, s13, qw2, s2)
        results.append((out64, out_bf16))
        x = (out_bf16.astype(np.uint32) << 16).view(np.float32)
    return results
