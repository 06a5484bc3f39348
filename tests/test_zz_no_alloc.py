"""fp8_linear_noalloc (the quantised input in the library's static device
scratch) against fp8_linear (the same path with a caller workspace): bit for
bit, on two calls in a row, the second with a smaller input, so the second
call reuses the scratch the first one filled. Also the paths that need no
scratch (default maths, the single-launch kernel) and the size limit."""
import numpy as np
import pytest

import synth
from gpu_util import bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import w8a8_fp8_linear_amd as w8  # noqa: E402


def _layer(M, N, K, seed):
    d = synth.dense_workload(M=M, N=N, K=K, n_outlier=max(1, K // 100), seed=seed)
    x = to_dev_bf16(d["x"])
    wq, ws = w8.quantize_weight(to_dev_bf16(d["w"]))
    return x, wq, ws


def test_noalloc_equals_fp8_linear_two_calls():
    for M, N, K, seed in [(4096, 6144, 2048, 0), (300, 1040, 1024, 1)]:
        print(f"[noalloc] M={M} N={N} K={K}", flush=True)
        x, wq, ws = _layer(M, N, K, seed)
        ref = w8.fp8_linear(x, wq, ws)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        got = w8.fp8_linear_noalloc(x, wq, ws, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert np.array_equal(bf16_bits(got), bf16_bits(ref)), f"M={M}: differs from fp8_linear"


@pytest.mark.parametrize("M,fast_math", [(4, True), (12, True), (40, False)])
def test_noalloc_paths_without_scratch(M, fast_math):
    x, wq, ws = _layer(M, 1040, 528, 2)
    ref = w8.fp8_linear(x, wq, ws, fast_math=fast_math)
    got = w8.fp8_linear_noalloc(x, wq, ws, fast_math=fast_math)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(got), bf16_bits(ref))


def test_noalloc_size_limit():
    x = torch.zeros((8192, 8192), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((16, 8192), dtype=torch.uint8, device="cuda")
    ws = torch.ones(16, dtype=torch.float32, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:
        w8.fp8_linear_noalloc(x, wq, ws)
    assert e.value.status == 8


def test_noalloc_at_the_scratch_limit():
    """The largest input the scratch holds: 16368 x 4096 codes (align256 of
    M*K) and 16368 scales (align256 of 4*M) fill the 64 MiB array to its last
    byte; bit for bit against fp8_linear. One row more is refused."""
    K, N = 4096, 48
    limit = int(w8.lib().fp8_linear_noalloc_max_bytes())
    M = 16368
    assert int(w8.lib().fp8_linear_workspace_bytes(M, K)) == limit
    assert int(w8.lib().fp8_linear_workspace_bytes(M + 1, K)) > limit
    print(f"[noalloc] M={M} K={K} at the scratch limit", flush=True)
    x, wq, ws = _layer(M, N, K, 3)
    ref = w8.fp8_linear(x, wq, ws)
    got = w8.fp8_linear_noalloc(x, wq, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(got), bf16_bits(ref))
    x1 = torch.zeros((M + 1, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:
        w8.fp8_linear_noalloc(x1, wq, ws)
    assert e.value.status == 8


def test_noalloc_in_a_hip_graph():
    """The callers this entry point is for: captured once into a HIP graph and
    replayed three times; before each replay an eager call on another input
    overwrites the shared scratch. Every replay must equal fp8_linear bit for
    bit (the captured quantisation rewrites the scratch it then reads)."""
    x, wq, ws = _layer(300, 1040, 1024, 4)
    x2, _, _ = _layer(700, 1040, 1024, 5)
    ref = bf16_bits(w8.fp8_linear(x, wq, ws))
    out = torch.empty((300, 1040), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((700, 1040), dtype=torch.bfloat16, device="cuda")
    w8.fp8_linear_noalloc(x, wq, ws, out=out)  # eager first: the scratch address is looked up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.fp8_linear_noalloc(x, wq, ws, out=out)
    for i in range(3):
        out.zero_()
        w8.fp8_linear_noalloc(x2, wq, ws, out=out2)   # eager work that overwrites the scratch
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out), ref), f"replay {i} differs"
