"""bench.py's command line on the CPU: it measures one GPU and refuses --gpus N > 1 before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2, res
    assert "measures one GPU" in res.stderr and "--gpus 2" in res.stderr, res.stderr
    assert res.stdout == "", res.stdout  # no JSON line


def test_prefill_parity_report():
    """The bench line's parity figures: zero for the oracle's own BF16 output,
    and a planted one-ulp flip and a large error counted as the criterion
    defines them (against 1e-2 rms of the exact result)."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench
    import oracle
    import synth

    d = synth.dense_workload(**synth.DENSE_SMALL, seed=0)
    qx, sx, _ = oracle.quantize_rows(synth.bf16_bits_to_f32(d["x"]))
    qw, sw, _ = oracle.quantize_rows(synth.bf16_bits_to_f32(d["w"]))
    y64, ybf = oracle.w8a8_linear(qx, sx, qw, sw)
    rep = bench._parity_prefill(ybf.copy(), y64, ybf)
    assert rep["frobenius"] == 0 and rep["max_abs_over_rms"] == 0 and rep["n_over_1e-2_rms"] == 0
    assert rep["frobenius_met"] and rep["max_abs_met"] and rep["n_differ_from_oracle_bf16"] == 0
    bad = ybf.copy()
    bad.flat[0] ^= 1                                   # one ulp: far below 1e-2 rms for this element
    i = int(np.argmax(np.abs(y64)))
    bad.flat[i] = oracle.round_to_bf16_bits(np.array([y64.flat[i] * 2.0]))[0]  # a doubled value
    rep = bench._parity_prefill(bad, y64, ybf)
    assert rep["n_differ_from_oracle_bf16"] == 2 and rep["n_over_1e-2_rms"] == 1 and not rep["max_abs_met"]
