"""Pins of the oracle's E4M3 codec against the format's definition.

The codec is checked against values fixed by the E4M3 format (golden files),
against torch's float8_e4m3fn (a library implementation of the same format),
by the exact round trip of every finite code, by monotonicity, and by a
second encoder written on the float32 bit fields, over every float32 near a
rounding boundary and a strided sweep of all float32 patterns.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_decode_golden_values():
    for code, val in _read_rows("e4m3_values.txt"):
        got = oracle.decode(np.array([int(code, 16)], np.uint8))[0]
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_table()
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin]))


def test_format_constants():
    t = oracle.decode_table()
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert oracle.finite_codes().size == 254
    mags = oracle.magnitudes()
    assert mags.size == 127 and mags[1] == 2.0 ** -9 and mags[-1] == 448.0
    assert set(np.flatnonzero(np.isnan(t))) == {0x7F, 0xFF}


def test_roundtrip_every_finite_code():
    codes = oracle.finite_codes()
    vals = oracle.decode(codes).astype(np.float32)
    assert np.array_equal(oracle.encode(vals), codes)
    assert np.array_equal(oracle.encode_bits(vals), codes)


def test_encode_golden_cases():
    for val, code, *_ in _read_rows("e4m3_encode_cases.txt"):
        v = np.array([float(val)], np.float32)
        assert oracle.encode(v)[0] == int(code, 16), val
        assert oracle.encode_bits(v)[0] == int(code, 16), val


def test_encode_monotone():
    v = np.sort(np.random.default_rng(1).uniform(-470, 470, 200000).astype(np.float32))
    dec = oracle.decode(oracle.encode(v))
    assert np.all(np.diff(dec) >= 0)


def _boundary_neighbourhood(span=1024):
    """Every float32 within ``span`` ulps of each E4M3 value and midpoint."""
    mags = oracle.magnitudes()
    pts = np.concatenate([mags, (mags[:-1] + mags[1:]) / 2, [464.0, 2.0 ** -10]])
    pts = pts.astype(np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    off = np.arange(-span, span + 1, dtype=np.int64)
    allb = (bits[:, None] + off[None, :]).reshape(-1)
    allb = allb[(allb >= 0) & (allb < 0x7F800000)]
    v = allb.astype(np.uint32).view(np.float32)
    return np.concatenate([v, -v])


def test_encode_matches_torch_near_boundaries():
    v = _boundary_neighbourhood()
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(v), ref)


def test_encode_matches_torch_random():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-12, 6, 2_000_000))).astype(np.float32)
    v = v[np.abs(v) < 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(v), ref)


def test_two_encoders_agree_near_boundaries():
    v = _boundary_neighbourhood(span=4096)
    assert np.array_equal(oracle.encode(v), oracle.encode_bits(v))


def test_two_encoders_agree_strided_sweep():
    # one float32 pattern in every 1021, covering every exponent and sign
    bits = np.arange(0, 1 << 32, 1021, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.encode(v), oracle.encode_bits(v))


def test_two_encoders_agree_all_bf16_patterns():
    v = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    v = v[~np.isnan(v)]
    assert np.array_equal(oracle.encode(v), oracle.encode_bits(v))


@pytest.mark.slow
def test_two_encoders_agree_every_float32():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        v = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32).view(np.float32)
        v = v[~np.isnan(v)]
        assert np.array_equal(oracle.encode(v), oracle.encode_bits(v)), hex(start)


def test_saturation_and_sign():
    v = np.array([448.0, 449.0, 463.99, 464.0, 1e38, np.inf, -448.5, -np.inf], np.float32)
    assert list(oracle.encode(v)) == [0x7E] * 6 + [0xFE] * 2
    tiny = np.array([-1e-5, -0.0, -1e-45, 1e-45, 0.0], np.float32)
    assert list(oracle.encode(tiny)) == [0x80, 0x80, 0x80, 0x00, 0x00]


def test_decode_subnormal_spacing():
    t = oracle.decode_table()
    assert [t[c] for c in range(8)] == [m * 2.0 ** -9 for m in range(8)]
    assert e4m3.E4M3_MAX == 448.0
