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
