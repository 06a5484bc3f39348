"""Exhaustive device checks of the two conversions every bit-exact result
rests on.

* E4M3: every float32 bit pattern of magnitude <= 448, both signs, through
  the quantisers' final step (clamp to +-448, then the hardware conversion),
  against torch's CPU cast to float8_e4m3fn, which the oracle's encoder is
  pinned to; a strided sample is also compared with the oracle's own
  bit-field encoder. Magnitudes above 448 (the clamp) are covered on a
  sample: they must give +-448.
* BF16: every non-NaN float32 bit pattern through the BF16 rounding of every
  BF16 result, against torch's CPU cast (round to nearest even).

Inputs are generated on the device from bit-pattern ranges, chunk by chunk;
the expected codes are computed on the CPU.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import w8a8_fp8_linear_amd as w8  # noqa: E402

CHUNK = 1 << 26
E4M3_LAST = 0x43E00000          # 448.0
F32_INF = 0x7F800000


def _patterns(lo, hi):
    """float32 values with bit patterns lo .. hi-1 (non-negative), on the GPU."""
    return torch.arange(lo, hi, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)


def test_e4m3_every_float32_up_to_448():
    print("[convert] e4m3 over |v| <= 448", flush=True)
    n_checked = 0
    for lo in range(0, E4M3_LAST + 1, CHUNK):
        hi = min(lo + CHUNK, E4M3_LAST + 1)
        v = _patterns(lo, hi)
        got = w8.e4m3_from_f32(v)
        got_neg = w8.e4m3_from_f32(-v)
        want = v.cpu().to(torch.float8_e4m3fn).view(torch.uint8)
        got_c, got_neg_c = got.cpu(), got_neg.cpu()
        bad = torch.nonzero(got_c != want)
        assert bad.numel() == 0, f"{bad.numel()} codes differ in [{lo:#x}, {hi:#x}), first pattern {lo + int(bad[0]):#x}"
        # the sign is a separate bit of the format: -v encodes as code(v) | 0x80
        bad = torch.nonzero(got_neg_c != (want | 0x80))
        assert bad.numel() == 0, f"{bad.numel()} negative codes differ, first pattern {lo + int(bad[0]):#x}"
        # the oracle's bit-field encoder on a strided sample
        idx = np.arange(0, hi - lo, 4099)
        vals = v.cpu().numpy()[idx]
        assert np.array_equal(got_c.numpy()[idx], oracle.encode_bits(vals))
        assert np.array_equal(got_neg_c.numpy()[idx], oracle.encode_bits(-vals))
        n_checked += 2 * (hi - lo)
        del v, got, got_neg
    print(f"e4m3: {n_checked} float32 values, 0 mismatches", flush=True)


def test_e4m3_saturates_above_448():
    rng = np.random.default_rng(0)
    bits = rng.integers(E4M3_LAST + 1, F32_INF + 1, 1 << 20, dtype=np.int64).astype(np.uint32)
    v = torch.from_numpy(bits.view(np.float32)).cuda()
    got = w8.e4m3_from_f32(v).cpu().numpy()
    got_neg = w8.e4m3_from_f32(-v).cpu().numpy()
    assert np.all(got == 0x7E) and np.all(got_neg == 0xFE)


def test_bf16_every_float32():
    print("[convert] bf16 over every non-NaN float32", flush=True)
    n_checked = 0
    for lo in range(0, F32_INF + 1, CHUNK):
        hi = min(lo + CHUNK, F32_INF + 1)            # the non-NaN magnitudes: 0 .. +inf
        v = _patterns(lo, hi)
        for sign in (1.0, -1.0):
            x = v if sign > 0 else -v
            got = w8.bf16_from_f32(x).view(torch.int16).cpu()
            want = x.cpu().to(torch.bfloat16).view(torch.int16)
            bad = torch.nonzero(got != want)
            assert bad.numel() == 0, (f"{bad.numel()} BF16 results differ, sign {sign}, first pattern "
                                      f"{lo + int(bad[0]):#x}")
            n_checked += hi - lo
        del v
    print(f"bf16: {n_checked} float32 values, 0 mismatches", flush=True)


def test_conversion_ragged_lengths():
    """Lengths that are not a multiple of the 4 values a thread converts."""
    rng = np.random.default_rng(1)
    for n in (1, 2, 3, 5, 1023, 1025):
        x = (rng.standard_normal(n) * 100).astype(np.float32)
        v = torch.from_numpy(x).cuda()
        assert np.array_equal(w8.e4m3_from_f32(v).cpu().numpy(), oracle.encode_bits(np.clip(x, -448, 448)))
        got = w8.bf16_from_f32(v).view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.round_to_bf16_bits(x.astype(np.float64)))


@pytest.mark.parametrize("nbytes", [16, 32768, 16809984, 100016])
def test_read_probe_checksums(nbytes):
    """read_probe reads every byte: its per-32 KB XOR words match the host's."""
    rng = np.random.default_rng(nbytes)
    data = rng.integers(0, 256, nbytes, dtype=np.uint8)
    sink = w8.read_probe(torch.from_numpy(data).cuda()).cpu().numpy().view(np.uint32)
    padded = np.zeros(-(-nbytes // 32768) * 32768, np.uint8)
    padded[:nbytes] = data
    want = np.bitwise_xor.reduce(padded.view(np.uint32).reshape(-1, 8192), axis=1)
    assert np.array_equal(sink[:want.size], want)


def test_clock_probe_reads_a_plausible_clock():
    """clock_probe: every workgroup spans at least 400 ticks of the 100 MHz clock, and the shader
    clock it reports lies between 0.5 and 3 GHz (the chip's top clock is 2.4 GHz)."""
    print("[clock_probe] 256 workgroups", flush=True)
    out = w8.clock_probe(256)
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert (v[:, 1] >= 400).all() and (v[:, 1] < 100000).all(), v[:, 1].min()
    ghz = 0.1 * v[:, 0] / v[:, 1]
    assert (ghz > 0.5).all() and (ghz < 3.0).all(), (ghz.min(), ghz.max())
    assert abs(w8.clock_ghz(out) - float(np.median(ghz))) < 1e-9
    print("clock_probe median GHz", float(np.median(ghz)), flush=True)
