"""Oracle-side helpers for the MXFP4 expert parity tests (test infrastructure).

Everything here is composed from the oracle's definitions (MX quantiser,
exact dequantisation, SwiGLU); nothing comes from the GPU path except the
arrays under test.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from gpu_util import MFMA_GROUP_ERR, U32, map_row_chunks
from moe_util import swiglu_bound


def mx_quantize_chunked(x, rows=2048):
    """oracle.mx_quantize_rows over row chunks (bounded temporary memory, chunks
    on a thread pool)."""
    res = map_row_chunks(oracle.mx_quantize_rows, x, rows)
    return np.concatenate([q for q, _ in res]), np.concatenate([s for _, s in res])


def quantized_mx_moe(T, H, I, E, k, n_outlier=0, passes=1, seed=0):
    """Seeded inputs with tokens and weights quantised to MXFP4 by the oracle."""
    d = synth.moe_workload(T=T, H=H, I=I, E=E, k=k, n_outlier=n_outlier, passes=passes, seed=seed)
    q13, s13 = mx_quantize_chunked(synth.bf16_bits_to_f32(d["w13"].reshape(E * 2 * I, H)))
    q2, s2 = mx_quantize_chunked(synth.bf16_bits_to_f32(d["w2"].reshape(E * H, I)))
    x32 = synth.bf16_bits_to_f32(d["x"])
    qx, sx = mx_quantize_chunked(x32)
    return {
        "x_bits": d["x"], "x32": x32, "qx": qx, "sx": sx, "routes": d["routes"],
        "q13": q13.reshape(E, 2 * I, H // 2), "s13": s13.reshape(E, 2 * I, H // 32),
        "q2": q2.reshape(E, H, I // 2), "s2": s2.reshape(E, H, I // 32),
        "T": T, "H": H, "I": I, "E": E, "k": k,
    }


def mx_bound(a, b, K):
    """Per-element bound on |gpu32 - exact| of an FP4 matrix-core product a . b^T
    (dequantised operands): the MFMA's own summation (as for the E4M3 path:
    each 128-deep instruction within 2**-10 of its sum of |terms|) plus one
    float32 rounding per instruction and a few for the epilogue."""
    return (MFMA_GROUP_ERR + (K / 128 + 3) * U32) * 1.01 * (np.abs(a) @ np.abs(b).T)


def sorted_rows_gate_up(qx, sx, ids, perm, rows, q13, s13, k):
    """Exact gate/up values of sorted rows ``rows`` and their error bound."""
    rows = np.asarray(rows)
    slots = np.asarray(perm)[rows]
    tok = slots // k
    exp = np.asarray(ids).reshape(-1)[slots]
    H = 2 * qx.shape[1]
    gu = np.zeros((rows.size, q13.shape[1]))
    err = np.zeros_like(gu)
    for e in np.unique(exp):
        sel = np.flatnonzero(exp == e)
        a = oracle.mx_dequant(qx[tok[sel]], sx[tok[sel]])
        b = oracle.mx_dequant(q13[e], s13[e])
        gu[sel] = a @ b.T
        err[sel] = mx_bound(a, b, H)
    return gu, err


def _block_codes(amax):
    """E8M0 byte of blocks with the given exact maxima (the oracle's rule)."""
    amax = np.asarray(amax, np.float64)
    out = np.full(amax.shape, 127, np.int64)
    nz = amax > 0
    _, ex = np.frexp(amax[nz])
    out[nz] = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127) + 127
    return out


def check_mx_requant(qh_gpu, sh_gpu, gu64, gu_err):
    """Explainable-difference check of MXFP4 h rows against the oracle.

    The oracle quantises h = fl32(silu(g) * u) of its exact gate/up values.
    The GPU's g, u lie within ``gu_err``; swiglu_bound carries that to a
    bound dh on the GPU's h.
    Then (a) a block's E8M0 byte must lie between the bytes of the block
    maxima of |h| - dh and |h| + dh, and (b) under the GPU's own block
    scale, each code must decode inside [dec(enc(v - dv)), dec(enc(v + dv))]
    with v, dv the value and its bound in units of that scale. So a code or
    a scale may differ from the oracle's only where the oracle's value lies
    within the propagated error of a rounding or binade boundary.
    """
    I = gu64.shape[1] // 2
    h32, dh = swiglu_bound(gu64, gu_err)
    h32 = h32.astype(np.float64)
    q_ref, s_ref = oracle.mx_quantize_rows(h32.astype(np.float32))
    n, nb = h32.shape[0], I // 32
    hb, db = np.abs(h32).reshape(n, nb, 32), dh.reshape(n, nb, 32)
    lo_code = _block_codes(np.maximum(hb - db, 0).max(axis=2))
    hi_code = _block_codes((hb + db).max(axis=2))
    s_gpu = np.asarray(sh_gpu, np.int64)
    bad_s = (s_gpu < np.minimum(lo_code, hi_code)) | (s_gpu > np.maximum(lo_code, hi_code))
    assert not bad_s.any(), f"{bad_s.sum()} block scales outside the explainable range"
    scale = np.repeat(oracle.e8m0_value(s_gpu), 32, axis=1)
    v, dv = h32 / scale, dh / scale
    lo = oracle.e2m1_decode(oracle.e2m1_encode(v - dv))
    hi = oracle.e2m1_decode(oracle.e2m1_encode(v + dv))
    got = oracle.e2m1_decode(oracle.mx_unpack(np.asarray(qh_gpu, np.uint8)))
    bad = (got < np.minimum(lo, hi)) | (got > np.maximum(lo, hi))
    n_diff = int((np.asarray(qh_gpu) != q_ref).sum())
    assert not bad.any(), f"{bad.sum()} codes outside the explainable range (of {n_diff} differing bytes)"
    return {"n_values": int(h32.size), "n_code_bytes_differ": n_diff,
            "n_scales_differ": int((s_gpu != s_ref).sum()), "n_blocks": int(s_ref.size),
            "n_near_boundary": int((lo != hi).sum())}


def down_combine_ref(qh, sh, perm, ids, tw, q2, s2, k, tokens):
    """Exact down projection + combine for ``tokens`` from sorted MXFP4 h rows
    (the router-weighted copies summed at full precision, the value the GPU
    rounds once to BF16), and a bound on |out_gpu - out64| before that
    rounding: per copy the FP4 matrix-core bound, then the float32 rounding
    of each stored copy and of the float32 sum."""
    tokens = np.asarray(tokens)
    E, H, _ = q2.shape
    I = 2 * q2.shape[2]
    perm = np.asarray(perm)
    inv = np.full(ids.size, -1, np.int64)
    nv = int((perm >= 0).sum())
    inv[perm[:nv]] = np.arange(nv)
    out = np.zeros((tokens.size, H))
    err = np.zeros((tokens.size, H))
    absout = np.zeros((tokens.size, H))
    flat_ids = np.asarray(ids).reshape(-1)
    w = np.asarray(tw, np.float32).reshape(-1).astype(np.float64)
    for j in range(k):
        slots = tokens * k + j
        rows = inv[slots]
        valid = rows >= 0
        for e in np.unique(flat_ids[slots[valid]]):
            sel = np.flatnonzero(valid & (flat_ids[slots] == e))
            a = oracle.mx_dequant(qh[rows[sel]], sh[rows[sel]])
            b = oracle.mx_dequant(q2[e], s2[e])
            wt = w[slots[sel]][:, None]
            y = wt * (a @ b.T)
            ey = np.abs(wt) * mx_bound(a, b, I)
            out[sel] += y
            absout[sel] += np.abs(y)
            err[sel] += ey
    err += (k + 2) * U32 * 1.01 * absout
    return out, err
