"""GPU parity of the default maths (W8A16) and of fp8_linear's dispatch.

* w8a16_gemm on ragged, decode and full prefill shapes: every element inside
  the BF16 matrix-core bound (tests/gpu_util.w8a16_report), normalised
  Frobenius <= 4e-3.
* Single products are bit-exact: a one-hot BF16 row against every finite
  E4M3 code, through both kernels (pins operand roles, the E4M3 widening and
  the output layout).
* fp8_linear takes the FP8 path (quantize_per_token + w8a8_gemm, bit for bit)
  only with fast_math and more than 8 tokens, and the default maths otherwise.
* fp8_linear_single_launch (the quantisation fused into the decode GEMM,
  M <= 32, K <= 2048) is bit-identical to the two-launch chain, on workload
  rows and on zero, subnormal, huge and tie rows, and inside the E4M3 bound.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits, record, to_dev, to_dev_bf16, w8a16_report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import w8a8_fp8_linear_amd as w8  # noqa: E402


def _weights(d):
    qw, sw, _ = oracle.quantize_rows(synth.bf16_bits_to_f32(d["w"]))
    return qw, sw


def _run(x_bits, qw, sw):
    y = w8.w8a16_gemm(to_dev_bf16(x_bits), to_dev(qw), to_dev(sw))
    torch.cuda.synchronize()
    return bf16_bits(y)


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (5, 48, 528), (8, 8192, 2048), (17, 4096, 2048), (32, 1040, 272),
                                   (33, 1040, 272), (300, 6144, 128), (1000, 528, 1040), (513, 1040, 2064)])
def test_w8a16_parity(M, N, K):
    print(f"[w8a16] {M}x{N}x{K}", flush=True)
    d = synth.dense_workload(M=M, N=N, K=K, n_outlier=min(3, K), seed=M + N + K)
    qw, sw = _weights(d)
    got = _run(d["x"], qw, sw)
    rep = w8a16_report(got, d["x"], qw, sw)
    record(f"w8a16 {M}x{N}x{K}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep


def test_w8a16_prefill_full():
    """4096 x 2048 -> 6144, the tiled kernel at the benchmark's shape: every output."""
    d = synth.dense_workload(**synth.DENSE_PREFILL, seed=0)
    qw, sw = _weights(d)
    got = _run(d["x"], qw, sw)
    rep = w8a16_report(got, d["x"], qw, sw)
    print("w8a16 prefill", rep, flush=True)
    record("w8a16 prefill 4096x2048->6144 (full)", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep


@pytest.mark.parametrize("M", [256, 16])
def test_w8a16_every_code_single_product_exact(M):
    codes = oracle.finite_codes()
    K = 64
    vals = np.array([1.0, -0.75, 3.0, 2.0 ** -7], np.float32)
    x = np.zeros((M, K), np.uint16)
    for m in range(M):
        x[m, m % K] = (vals[m % vals.size:m % vals.size + 1].view(np.uint32) >> 16).astype(np.uint16)[0]
    qw = np.zeros((codes.size, K), np.uint8)
    for n in range(codes.size):
        qw[n, :] = codes[n]                       # every K position holds the same code
    N = (codes.size + 15) // 16 * 16
    qw = np.concatenate([qw, np.zeros((N - codes.size, K), np.uint8)])
    sw = np.ones(N, np.float32)
    got = _run(x, qw, sw)
    _, want = oracle.w8a16_linear(x, qw, sw)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("K", [1024, 4096])
def test_fp8_linear_dispatch(K):
    # M > 8 with fast maths: the FP8 chain, as one fused launch for M <= 16 and K <= 2048 and as
    # quantisation + GEMM otherwise; both must give the bits of quantize_per_token + w8a8_gemm
    d = synth.dense_workload(M=64, N=1040, K=K, n_outlier=8, seed=3)
    qw, sw = _weights(d)
    wq, ws = to_dev(qw), to_dev(sw)
    for M in (64, 32, 17, 16, 12, 9, 8, 1):
        print(f"[fp8_linear dispatch] M={M} K={K}", flush=True)
        x = to_dev_bf16(d["x"][:M])
        fast = bf16_bits(w8.fp8_linear(x, wq, ws, fast_math=True))
        slow = bf16_bits(w8.fp8_linear(x, wq, ws, fast_math=False))
        ref8 = bf16_bits(w8.w8a8_linear(x, wq, ws))
        ref16 = bf16_bits(w8.w8a16_gemm(x, wq, ws))
        torch.cuda.synchronize()
        assert np.array_equal(slow, ref16), M
        assert np.array_equal(fast, ref8 if M > 8 else ref16), M


def test_w8a16_argument_errors():
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((16, 24), dtype=torch.uint8, device="cuda")
    s = torch.ones(16, dtype=torch.float32, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:
        w8.w8a16_gemm(x, w, s)                    # K = 24 is not a multiple of 16
    assert e.value.status == 4


def _special_decode_rows(M, K, rng):
    """Rows that exercise the quantiser: zero, subnormal, tiny-negative, huge, ties of the E4M3 grid."""
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-10, 10, (M, 1)))).astype(np.float32)
    x[0] = 0.0
    if M > 1:
        x[1] = 0.0
        x[1, K // 3] = 3e-39                            # subnormal row maximum
        x[1, 0] = -1e-40
    if M > 2:
        x[2, :] = 448.0 * np.sign(rng.standard_normal(K))
        x[2, 5] = 3.38e38                              # near the largest BF16
    if M > 3:
        x[3, :] = rng.choice([0.5, 1.0625, 1.1875, -2.0625, 3.1e-3], K)   # E4M3 ties after scaling
    return oracle.round_to_bf16_bits(x)


@pytest.mark.parametrize("M,N,K", [(1, 8192, 2048), (9, 8192, 2048), (16, 8192, 2048), (17, 8192, 2048),
                                   (32, 8192, 2048), (13, 1040, 528), (24, 16, 16), (31, 48, 2048),
                                   (12, 4096, 1024)])
def test_single_launch_equals_chain(M, N, K):
    """fp8_linear_single_launch is bit-identical to quantize_per_token + w8a8_gemm, and
    inside the E4M3 matrix-core bound against the oracle."""
    print(f"[fused decode] {M}x{N}x{K}", flush=True)
    rng = np.random.default_rng(M * 7 + K)
    d = synth.dense_workload(M=M, N=N, K=K, n_outlier=min(3, K), seed=M + N + K)
    qw, sw = _weights(d)
    wq, ws = to_dev(qw), to_dev(sw)
    for bits in (d["x"], _special_decode_rows(M, K, rng)):
        x = to_dev_bf16(bits)
        fused = bf16_bits(w8.fp8_linear_single_launch(x, wq, ws))
        q, s = w8.quantize_per_token(x)
        chain = bf16_bits(w8.w8a8_gemm(q, s, wq, ws))
        torch.cuda.synchronize()
        assert np.array_equal(fused, chain)
    from gpu_util import gemm_report
    x32 = synth.bf16_bits_to_f32(d["x"])
    qx, sx, _ = oracle.quantize_rows(x32)
    fused = bf16_bits(w8.fp8_linear_single_launch(to_dev_bf16(d["x"]), wq, ws))
    torch.cuda.synchronize()
    rep = gemm_report(fused, qx, sx, qw, sw)
    record(f"fp8_linear_single_launch {M}x{N}x{K}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep
