#!/usr/bin/env python3
"""Benchmark of the W8A8 FP8 linear path on one MI355X.

A step is one pass of the prefill projection: per-token FP8 quantisation of
a 4096 x 2048 BF16 activation followed by the scaled FP8 GEMM against a
[6144 x 2048] E4M3 weight (per-output-row scales) with a BF16 output. The
weight is quantised once, before timing. Inputs are seeded synthetic data
resident in HBM before the timed region starts.

Printed: one JSON line. ``value`` is the step's throughput in TFLOP/s
(2*M*N*K per step over the wall time of the timed steps). ``roofline``
describes the dominant kernel (the GEMM) against the FP8 MFMA dense peak,
using HIP event timing of each GEMM launch on the stream it runs on.
``decode`` reports the weight-streaming GEMM at M = 8 (and 1, 32) as HBM
GB/s with a rotation of distinct weight buffers larger than the last-level
cache. ``cpu_baseline`` is the CPU oracle timed on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
METRIC = "W8A8 TFLOP/s & % FP8 MFMA peak (prefill M=4096); HBM GB/s at decode M=8"


def _bf16_dev(bits):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bench_prefill(steps, warmup):
    import torch

    import synth
    import w8a8_fp8_linear_amd as w8

    cfg = synth.DENSE_PREFILL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    d = synth.dense_workload(**cfg, seed=0)
    x = _bf16_dev(d["x"])
    wq, ws = w8.quantize_weight(_bf16_dev(d["w"]))
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        w8.quantize_per_token(x, xq, xs)
        if ev is not None:
            ev[0].record(stream)
        w8.w8a8_gemm(xq, xs, wq, ws, out=y)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gemm_ms = sorted(a.elapsed_time(b) for a, b in evs)
    gemm_avg = sum(gemm_ms) / len(gemm_ms)

    # quantiser alone, same stream, event-timed
    qe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in qe:
        a.record(stream)
        w8.quantize_per_token(x, xq, xs)
        b.record(stream)
    torch.cuda.synchronize()
    q_avg = sum(a.elapsed_time(b) for a, b in qe) / steps

    flops = 2.0 * M * N * K
    gemm_bytes = M * K + N * K + 2 * M * N + 4 * (M + N)
    q_bytes = 2 * M * K + M * K + 4 * M
    return {
        "M": M, "N": N, "K": K, "wall_s": wall, "ms_per_step": 1e3 * wall / steps,
        "tflops": flops * steps / wall / 1e12,
        "gemm_ms_avg": gemm_avg, "gemm_ms_p10": gemm_ms[len(gemm_ms) // 10],
        "gemm_ms_p90": gemm_ms[(9 * len(gemm_ms)) // 10],
        "gemm_tflops": flops / (gemm_avg * 1e-3) / 1e12, "gemm_flops": flops, "gemm_bytes": gemm_bytes,
        "quant_ms_avg": q_avg, "quant_gbs": q_bytes / (q_avg * 1e-3) / 1e9, "quant_bytes": q_bytes,
        "tokens_per_s": M * steps / wall,
    }


def bench_decode(Ms=(8, 1, 32), n_buffers=40, reps=5):
    import torch

    import synth
    import w8a8_fp8_linear_amd as w8

    cfg = synth.DENSE_DECODE
    N, K = cfg["N"], cfg["K"]
    # distinct weight buffers: 40 x 16.8 MB = 671 MB, more than the last-level cache
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    wqs, wss = [], []
    d = synth.dense_workload(M=1, K=K, N=N, seed=0)
    wq0, ws0 = w8.quantize_weight(_bf16_dev(d["w"]))
    for i in range(n_buffers):
        wqs.append(wq0.roll(i, dims=0).contiguous())
        wss.append(ws0.roll(i).contiguous())
    out = {}
    stream = torch.cuda.current_stream()
    for M in Ms:
        dm = synth.dense_workload(M=M, K=K, N=N, seed=1)
        x = _bf16_dev(dm["x"])
        xq, xs = w8.quantize_per_token(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        for i in range(n_buffers):
            w8.w8a8_gemm(xq, xs, wqs[i], wss[i], out=y)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_buffers * reps)]
        t0 = time.perf_counter()
        for j, (a, b) in enumerate(evs):
            a.record(stream)
            w8.w8a8_gemm(xq, xs, wqs[j % n_buffers], wss[j % n_buffers], out=y)
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        avg = sum(ms) / len(ms)
        wbytes = N * K + 4 * N
        out[f"M{M}"] = {
            "kernel_us_avg": 1e3 * avg, "kernel_us_p50": 1e3 * ms[len(ms) // 2],
            "weight_stream_GBs": wbytes / (avg * 1e-3) / 1e9,
            "frac_hbm_peak": wbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "wall_us_per_call": 1e6 * wall / len(evs), "weight_bytes": wbytes,
        }
    return out


def cpu_baseline():
    """The CPU oracle on the full prefill workload (activation quantisation,
    exact float64 GEMM, BF16 rounding), timed once on this host."""
    import numpy as np

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cfg = synth.DENSE_PREFILL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    d = synth.dense_workload(**cfg, seed=0)
    qw, sw, _ = oracle.quantize_rows(synth.bf16_bits_to_f32(d["w"]))
    x = synth.bf16_bits_to_f32(d["x"])
    t0 = time.perf_counter()
    qx, sx, _ = oracle.quantize_rows(x)
    oracle.w8a8_linear(qx, sx, qw, sw)
    dt = time.perf_counter() - t0
    return {"value": 2.0 * M * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full prefill workload {M}x{K} -> {N}: quantise + float64 GEMM + BF16 rounding, one run "
                      f"({dt:.2f} s)", "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path does not shard).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    print(f"[bench] prefill: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    pre = bench_prefill(args.steps, args.warmup)
    dec = None
    if not args.no_decode:
        print("[bench] decode", file=sys.stderr, flush=True)
        dec = bench_decode()
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline()
    achieved = pre["gemm_flops"] / (pre["gemm_ms_avg"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(pre["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> fp32 acc -> bf16",
        "data": "synthetic (seeded N(0,1) activations with 1% x20 outlier channels, N(0,0.02) weights)",
        "config": {"workload": "prefill projection 4096 tokens x 2048 -> 6144 (per-token quant + W8A8 GEMM)",
                   "M": pre["M"], "N": pre["N"], "K": pre["K"]},
        "roofline": {"bound": "mfma", "kernel": "gemm_tiled<256,192>", "achieved": round(achieved, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": None},
        "gemm_us_avg": round(pre["gemm_ms_avg"] * 1e3, 3),
        "gemm_us_p10_p90": [round(pre["gemm_ms_p10"] * 1e3, 3), round(pre["gemm_ms_p90"] * 1e3, 3)],
        "quant_us_avg": round(pre["quant_ms_avg"] * 1e3, 3),
        "quant_GBs": round(pre["quant_gbs"], 1),
        "tokens_per_s": round(pre["tokens_per_s"], 1),
        "decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
