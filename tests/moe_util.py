"""Oracle-side helpers for the routed-expert parity tests (test infrastructure).

Everything here is composed from the oracle's own definitions (decode,
exact dequantised sums, SwiGLU, the per-row quantiser); nothing comes from
the GPU path except the arrays under test.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from gpu_util import MFMA_GROUP_ERR, U32, bf16_ulp, map_row_chunks

SILU_DERIV_MAX = 1.1  # max |d silu / dg| over the reals is ~1.0998


def quantized_moe(T, H, I, E, k, n_outlier=0, passes=1, seed=0):
    """Seeded inputs with weights quantised by the oracle (the reference codes)."""
    d = synth.moe_workload(T=T, H=H, I=I, E=E, k=k, n_outlier=n_outlier, passes=passes, seed=seed)
    q13, s13 = _quant_rows_chunked(synth.bf16_bits_to_f32(d["w13"].reshape(E * 2 * I, H)))
    q2, s2 = _quant_rows_chunked(synth.bf16_bits_to_f32(d["w2"].reshape(E * H, I)))
    x32 = synth.bf16_bits_to_f32(d["x"])
    qx, sx, _ = oracle.quantize_rows(x32)
    return {
        "x_bits": d["x"], "x32": x32, "qx": qx, "sx": sx, "routes": d["routes"],
        "q13": q13.reshape(E, 2 * I, H), "s13": s13.reshape(E, 2 * I),
        "q2": q2.reshape(E, H, I), "s2": s2.reshape(E, H), "T": T, "H": H, "I": I, "E": E, "k": k,
    }


def _quant_rows_chunked(x, rows=8192):
    """oracle.quantize_rows over row chunks (chunks on a thread pool)."""
    res = map_row_chunks(oracle.quantize_rows, x, rows)
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def sorted_rows_gate_up(qx, sx, ids, perm, rows, q13, s13, k):
    """Oracle gate/up values of sorted rows ``rows`` (perm = the exact sorted order).

    Returns (gu64 [n, 2I], err [n, 2I]) where err bounds |gu_gpu32 - gu64| for the
    E4M3 matrix-core path (see gpu_util.gemm_report).
    """
    rows = np.asarray(rows)
    slots = np.asarray(perm)[rows]
    tok = slots // k
    exp = np.asarray(ids).reshape(-1)[slots]
    n2I = q13.shape[1]
    H = qx.shape[1]
    gu = np.zeros((rows.size, n2I))
    err = np.zeros((rows.size, n2I))
    for e in np.unique(exp):
        sel = np.flatnonzero(exp == e)
        a = oracle.decode(qx[tok[sel]])
        b = oracle.decode(q13[e])
        scale = sx[tok[sel]].astype(np.float64)[:, None] * s13[e].astype(np.float64)[None, :]
        gu[sel] = scale * (a @ b.T)
        err[sel] = (MFMA_GROUP_ERR + (H / 64 + 3) * U32) * 1.01 * scale * (np.abs(a) @ np.abs(b).T)
    return gu, err


def swiglu_bound(gu64, gu_err):
    """The oracle's h = fl32(silu(g) * u) of exact gate/up rows, and a bound dh
    on a GPU's float32 h whose g, u are within ``gu_err``: the derivative
    bound of silu times the error of g, the error of u, and 2**-19 relative
    for the float32 evaluation with a fast exponential. Returns (h, dh)."""
    I = gu64.shape[1] // 2
    g, u = gu64[:, :I], gu64[:, I:]
    dg, du = gu_err[:, :I], gu_err[:, I:]
    silu = g / (1.0 + np.exp(-g))
    h32 = oracle.swiglu_f32(gu64)
    dh = SILU_DERIV_MAX * dg * (np.abs(u) + du) + np.abs(silu) * du + 2.0 ** -19 * np.abs(h32) + 1e-30
    return h32, dh


def check_requant(qh_gpu, sh_gpu, gu64, gu_err):
    """Explainable-flip check of requantised h rows against the oracle.

    The oracle quantises h = fl32(silu(g) * u) of its exact gate/up values.
    The GPU's g, u differ by at most ``gu_err``; that bound is carried through
    silu * u (plus float32 evaluation error) to a bound dh on h, to a bound
    on the row scale, and to a bound dv on the scaled value v = h / s. A GPU
    code must then decode inside [dec(enc(v - dv)), dec(enc(v + dv))], so it
    equals the oracle's code unless v lies within dv of a rounding boundary.
    Returns a dict of statistics; raises AssertionError on a violation.
    """
    h32, dh = swiglu_bound(gu64, gu_err)
    q_ref, s_ref, v_ref = oracle.quantize_rows(h32)
    # scale: amax moves by at most max dh of the row
    ds = np.max(dh, axis=1) / 448.0 + 2.0 ** -22 * s_ref
    s_gpu = np.asarray(sh_gpu, np.float64)
    bad_s = np.abs(s_gpu - s_ref) > ds
    assert not bad_s.any(), f"{bad_s.sum()} scales outside the bound"
    s = s_ref.astype(np.float64)[:, None]
    dv = dh / s + np.abs(h32) * (ds[:, None] / s) / s * 1.01 + 2.0 ** -22 * np.abs(v_ref)
    lo = oracle.decode(oracle.encode((v_ref - dv).astype(np.float32)))
    hi = oracle.decode(oracle.encode((v_ref + dv).astype(np.float32)))
    got = oracle.decode(np.asarray(qh_gpu, np.uint8))
    bad = (got < np.minimum(lo, hi)) | (got > np.maximum(lo, hi))
    n_diff = int((np.asarray(qh_gpu) != q_ref).sum())
    near = lo != hi
    assert not bad.any(), f"{bad.sum()} codes outside the explainable range (of {n_diff} differing)"
    return {"n": int(q_ref.size), "n_codes_differ": n_diff, "n_near_boundary": int(near.sum()),
            "max_scale_rel_diff": float(np.max(np.abs(s_gpu - s_ref) / s_ref))}


def down_combine_ref(qh, sh, perm, ids, tw, q2, s2, k, tokens):
    """Oracle down projection + combine for ``tokens``, from sorted h codes.

    The router-weighted copies are summed at full precision (the value the
    GPU rounds once to BF16). Returns (out64 [n, H], err [n, H]); err bounds
    |out_gpu - out64| before the final BF16 rounding: per copy the E4M3
    matrix-core bound and the float32 scalings, then the float32 rounding of
    each stored copy and of the float32 sum.
    """
    tokens = np.asarray(tokens)
    E, H, I = q2.shape
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
            a = oracle.decode(qh[rows[sel]])
            b = oracle.decode(q2[e])
            scale = (sh[rows[sel]].astype(np.float64) * w[slots[sel]])[:, None] * s2[e].astype(np.float64)[None, :]
            y = scale * (a @ b.T)
            ey = (MFMA_GROUP_ERR + (I / 128 + 4) * U32) * 1.01 * scale * (np.abs(a) @ np.abs(b).T)
            out[sel] += y
            absout[sel] += np.abs(y)
            err[sel] += ey
    err += (k + 2) * U32 * 1.01 * absout
    return out, err


def bf16_compare(got_bits, ref64, err=None):
    """Frobenius / max-abs statistics of BF16 results against float64 references,
    and (if ``err`` is given) the count of elements outside err + half a BF16 ulp."""
    g = oracle.bf16_bits_to_f64(got_bits)
    ref_bf = oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(ref64))
    rms = float(np.sqrt(np.mean(ref64 ** 2)))
    diff = np.abs(g - ref_bf)
    rep = {
        "frobenius": float(np.linalg.norm(g - ref_bf) / max(np.linalg.norm(ref_bf), 1e-300)),
        "max_abs_over_rms": float(diff.max() / rms) if rms > 0 else 0.0,
        "n_over_1e-2_rms": int((diff > 1e-2 * rms).sum()),
        "n": int(g.size),
    }
    if err is not None:
        rep["n_bound_violations"] = int((np.abs(g - ref64) > err + 0.5 * bf16_ulp(g) + 1e-30).sum())
    return rep
