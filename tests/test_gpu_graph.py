"""The library under HIP graph capture: every entry point only enqueues
kernels on the caller's stream (no allocation, no memset, no host sync), so a
whole layer or routed-expert pass can be captured once and replayed. Each
graph is replayed several times with eager work of the program in between,
and every replay must equal the eager result bit for bit."""
import numpy as np
import pytest

from gpu_util import bf16_bits, to_dev, to_dev_bf16
from moe_util import quantized_moe

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import synth  # noqa: E402
import w8a8_fp8_linear_amd as w8  # noqa: E402


def _replays_match(run, expect, n=3):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = run()
    for i in range(n):
        torch.zeros(1 << 20, device="cuda").sum()          # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out), expect), f"replay {i} differs"


@pytest.mark.parametrize("fast_math,M", [(True, 512), (False, 512), (True, 24)])
def test_dense_layer_graph(fast_math, M):
    d = synth.dense_workload(M=M, N=1024, K=1024, n_outlier=4, seed=21)
    x = to_dev_bf16(d["x"])
    wq, ws = w8.quantize_weight(to_dev_bf16(d["w"]))
    wsp = torch.empty(max(int(w8.lib().fp8_linear_workspace_bytes(M, 1024)), 16), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, 1024), dtype=torch.bfloat16, device="cuda")
    eager = bf16_bits(w8.fp8_linear(x, wq, ws, fast_math=fast_math, workspace=wsp))
    torch.cuda.synchronize()
    _replays_match(lambda: w8.fp8_linear(x, wq, ws, fast_math=fast_math, out=y, workspace=wsp), eager)


def test_single_launch_graph():
    d = synth.dense_workload(M=24, N=1024, K=1024, n_outlier=4, seed=22)
    x = to_dev_bf16(d["x"])
    wq, ws = w8.quantize_weight(to_dev_bf16(d["w"]))
    y = torch.empty((24, 1024), dtype=torch.bfloat16, device="cuda")
    eager = bf16_bits(w8.fp8_linear_single_launch(x, wq, ws))
    torch.cuda.synchronize()
    _replays_match(lambda: w8.fp8_linear_single_launch(x, wq, ws, out=y), eager)


def test_moe_mxfp4_two_pass_graph():
    from mx_util import quantized_mx_moe
    d = quantized_mx_moe(T=301, H=384, I=384, E=9, k=4, n_outlier=3, passes=2, seed=29)
    routes = [(to_dev(i), to_dev(w)) for i, w in d["routes"]]
    q13, s13, q2, s2 = to_dev(d["q13"]), to_dev(d["s13"]), to_dev(d["q2"]), to_dev(d["s2"])
    x = to_dev_bf16(d["x_bits"])
    ws = w8.moe_mxfp4_workspace(d["T"], d["H"], d["I"], d["E"], d["k"])
    eager = [bf16_bits(o) for o in w8.moe_mxfp4_ffn(x, routes, q13, s13, q2, s2, workspace=ws)]
    torch.cuda.synchronize()
    outs = []

    def run():
        outs[:] = w8.moe_mxfp4_ffn(x, routes, q13, s13, q2, s2, workspace=ws)
        return outs[-1]

    _replays_match(run, eager[-1])
    assert np.array_equal(bf16_bits(outs[0]), eager[0])


def test_moe_two_pass_graph():
    d = quantized_moe(T=301, H=272, I=384, E=9, k=4, n_outlier=3, passes=2, seed=23)
    routes = [(to_dev(i), to_dev(w)) for i, w in d["routes"]]
    q13, s13, q2, s2 = to_dev(d["q13"]), to_dev(d["s13"]), to_dev(d["q2"]), to_dev(d["s2"])
    x = to_dev_bf16(d["x_bits"])
    ws = w8.moe_workspace(d["T"], d["H"], d["I"], d["E"], d["k"])
    eager = w8.moe_ffn(x, routes, q13, s13, q2, s2, workspace=ws)
    torch.cuda.synchronize()
    eager_bits = [bf16_bits(o) for o in eager]
    outs = []

    def run():
        outs[:] = w8.moe_ffn(x, routes, q13, s13, q2, s2, workspace=ws)
        return outs[-1]

    _replays_match(run, eager_bits[-1])
    assert np.array_equal(bf16_bits(outs[0]), eager_bits[0])
