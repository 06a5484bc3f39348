"""Pins of the oracle's per-row quantiser and BF16 rounding.

Quantiser: the amax element of every non-zero row lands on +-448; every
decoded value stays within +-448; a row made of 448 and every finite E4M3
value comes back exactly with scale 1; scaling a row by 2**j scales the
scale by 2**j and leaves the bytes alone; and, for rows [a, x] over every
finite BF16 x, the bytes equal torch's float8_e4m3fn cast of torch's
float32 quotient x / s (library division and library encoder).

BF16 rounding: single rounding from float64 (cases where rounding through
float32 first would differ), ties to even, subnormals and overflow, and
agreement with torch's float32 -> bfloat16 cast on float32 inputs.
"""
import numpy as np
import torch

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def _rows(seed=0, M=64, K=1024, n_out=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, n_out, replace=False)
    x[:, ch] *= 20
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def test_amax_maps_to_448():
    x = _rows()
    q, s, _ = oracle.quantize_rows(x)
    am = np.argmax(np.abs(x), axis=1)
    codes = q[np.arange(x.shape[0]), am]
    want = np.where(x[np.arange(x.shape[0]), am] < 0, 0xFE, 0x7E)
    assert np.array_equal(codes, want)
    assert np.all(np.abs(oracle.decode(q)) <= 448)


def test_amax_invariant_on_subnormal_and_extreme_rows():
    rows = []
    for a_bits in [0x0001, 0x0003, 0x007F, 0x0080, 0x7F7F, 0x3F80, 0x0A00]:
        xb = np.full(32, a_bits, np.uint16)
        xb[1::2] = 0
        xb[5] = a_bits | 0x8000
        rows.append(xb)
    x = bf16_bits_to_f32(np.stack(rows))
    q, s, _ = oracle.quantize_rows(x)
    for r in range(x.shape[0]):
        assert q[r, 0] == 0x7E and q[r, 5] == 0xFE
        assert s[r] > 0 and np.isfinite(s[r])


def test_exact_roundtrip_of_representable_row():
    codes = oracle.finite_codes()
    vals = oracle.decode(codes).astype(np.float32)
    row = np.concatenate([[448.0], vals]).astype(np.float32)[None, :]
    q, s, _ = oracle.quantize_rows(row)
    assert s[0] == 1.0
    assert q[0, 0] == 0x7E
    assert np.array_equal(q[0, 1:], codes)


def test_scale_invariance_powers_of_two():
    x = _rows(seed=3, M=16, K=256)
    q0, s0, _ = oracle.quantize_rows(x)
    for j in (-40, -7, -1, 1, 5, 30):
        q, s, _ = oracle.quantize_rows(x * np.float32(2.0 ** j))
        assert np.array_equal(q, q0), j
        assert np.array_equal(s, s0 * np.float32(2.0 ** j)), j


def test_zero_row():
    x = np.zeros((2, 16), np.float32)
    x[1, 3] = -0.0
    q, s, _ = oracle.quantize_rows(x)
    assert list(s) == [1.0, 1.0]
    assert q[0].sum() == 0 and q[1, 3] == 0x80


def _torch_quant_pair(a, x):
    """Bytes of x in the row [a, x] via torch's division and E4M3 cast."""
    at = torch.tensor(a, dtype=torch.float32)
    xt = torch.from_numpy(x)
    amax = torch.maximum(at.abs(), xt.abs())
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    v = xt / s
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), s.numpy()


def test_brute_force_every_bf16_against_torch():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x_all = bf16_bits_to_f32(allb)
    x_all = x_all[np.isfinite(x_all)]
    a_list = [1.0, 448.0, float(bf16_bits_to_f32(f32_to_bf16_bits(np.float32([3.7])))[0]),
              2.0 ** -120, float(bf16_bits_to_f32(np.uint16([0x0005]))[0]),
              float(bf16_bits_to_f32(np.uint16([0x7F7F]))[0])]
    for a in a_list:
        x = x_all[np.maximum(np.abs(x_all), abs(a)) > 0]
        row = np.stack([np.full_like(x, a), x], axis=1)
        q, s, _ = oracle.quantize_rows(row)
        ref, s_ref = _torch_quant_pair(a, x)
        assert np.array_equal(s, s_ref), a
        assert np.array_equal(q[:, 1], ref), a
        big = np.abs(x) > abs(a)
        assert np.all((q[big, 1] & 0x7F) == 0x7E), a


def test_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-80, 80, 1_000_000))).astype(np.float32)
    v = np.concatenate([v, np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_bf16_bits(v.astype(np.float64)), ref)


def test_bf16_single_rounding_from_float64():
    cases = {
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,   # above the tie: up (through float32 it would tie to 0x3F80)
        1.0 + 2.0 ** -8: 0x3F80,                # tie -> even
        1.0 + 3 * 2.0 ** -8: 0x3F82,            # tie -> even (up)
        -(1.0 + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** -133: 0x0001,                    # smallest subnormal
        2.0 ** -134: 0x0000,                    # tie with zero -> even
        3 * 2.0 ** -134: 0x0002,                # tie 1/2 -> even
        2.0 ** -134 + 2.0 ** -160: 0x0001,
        -1e-300: 0x8000,
        2.0 ** 128: 0x7F80,
        (2.0 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,  # tie between max and 2**128 -> even -> inf
        (2.0 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,  # largest finite
    }
    y = np.array(list(cases.keys()), np.float64)
    got = oracle.round_to_bf16_bits(y)
    assert [int(g) for g in got] == list(cases.values())
