"""Pins of the oracle's W8A8 linear layer.

* The float64 sums equal an int64 computation of the same sums (closed
  form: every product is an integer number of 2**-18 units), including the
  largest magnitudes at K = 2048.
* Brute force with exact rationals on small shapes: Y = bf16(s_x s_w sum
  dec * dec) computed with ``fractions.Fraction`` and rounded to BF16 by an
  integer nearest-even rule written here.
* Every pair of finite codes: a single-term product is representable in
  BF16, so Y equals dec(a) * dec(b) exactly (fixes operand roles and the
  E4M3 reading of both operands).
* Layout: a one-hot input row selects one column of the [out, in] weight.
"""
from fractions import Fraction

import numpy as np

import oracle
from oracle.linear import dequant_sum


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def test_int64_sums_equal_float64_sums():
    rng = np.random.default_rng(0)
    a = _rand_codes(rng, (37, 2048))
    b = _rand_codes(rng, (29, 2048))
    acc = dequant_sum(a, b)
    ints = oracle.w8a8_linear_int(a, b)
    assert np.array_equal(acc * 2.0 ** 18, ints.astype(np.float64))
    assert np.array_equal((acc * 2.0 ** 18).astype(np.int64), ints)


def test_largest_magnitudes_are_exact():
    a = np.full((2, 2048), 0x7E, np.uint8)
    b = np.full((3, 2048), 0x7E, np.uint8)
    b[1] = 0x01
    b[2, ::2] = 0xFE
    acc = dequant_sum(a, b)
    assert acc[0, 0] == 448.0 * 448.0 * 2048
    assert acc[0, 1] == 448.0 * 2.0 ** -9 * 2048
    assert acc[0, 2] == 0.0


def _bf16_rne_fraction(q: Fraction) -> float:
    """Nearest-even BF16 value of an exact rational (finite, normal range)."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128                      # 8 significant bits: 1.xxxxxxx
    n = int(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n, 128) * Fraction(2) ** e)


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(1)
    M, N, K = 3, 5, 48
    qx = _rand_codes(rng, (M, K))
    qw = _rand_codes(rng, (N, K))
    sx = rng.uniform(0.01, 3, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    dec = {c: Fraction(float(oracle.decode(np.uint8(c)))) for c in range(256) if (c & 0x7F) != 0x7F}
    _, ybf = oracle.w8a8_linear(qx, sx, qw, sw)
    got = oracle.bf16_bits_to_f64(ybf)
    for m in range(M):
        for n in range(N):
            acc = sum(dec[int(qx[m, k])] * dec[int(qw[n, k])] for k in range(K))
            want = _bf16_rne_fraction(Fraction(float(sx[m])) * Fraction(float(sw[n])) * acc)
            assert got[m, n] == want, (m, n)


def test_every_code_pair_single_term():
    codes = oracle.finite_codes()
    n = codes.size
    K = 16
    a = np.zeros((n, K), np.uint8)
    b = np.zeros((n, K), np.uint8)
    a[:, 0] = codes
    b[:, 0] = codes
    one = np.ones(n, np.float32)
    y64, ybf = oracle.w8a8_linear(a, one, b, one)
    d = oracle.decode(codes)
    want = np.outer(d, d)
    assert np.array_equal(y64, want)
    assert np.array_equal(oracle.bf16_bits_to_f64(ybf), want)


def test_one_hot_rows_select_weight_columns():
    rng = np.random.default_rng(2)
    M, N, K = 8, 12, 64
    qw = _rand_codes(rng, (N, K))
    sw = rng.uniform(0.5, 2, N).astype(np.float32)
    ks = rng.choice(K, M, replace=False)
    qx = np.zeros((M, K), np.uint8)
    qx[np.arange(M), ks] = 0x38            # 1.0
    sx = (2.0 ** rng.integers(-3, 4, M)).astype(np.float32)
    y64, _ = oracle.w8a8_linear(qx, sx, qw, sw)
    for m in range(M):
        want = sx[m].astype(np.float64) * sw.astype(np.float64) * oracle.decode(qw[:, ks[m]])
        assert np.array_equal(y64[m], want)


def test_power_of_two_scales_scale_output():
    rng = np.random.default_rng(3)
    qx = _rand_codes(rng, (4, 32))
    qw = _rand_codes(rng, (6, 32))
    sx = rng.uniform(0.1, 1, 4).astype(np.float32)
    sw = rng.uniform(0.1, 1, 6).astype(np.float32)
    y0, b0 = oracle.w8a8_linear(qx, sx, qw, sw)
    y1, b1 = oracle.w8a8_linear(qx, sx * np.float32(8), qw, sw * np.float32(0.25))
    assert np.array_equal(y1, y0 * 2)
    assert np.array_equal(oracle.bf16_bits_to_f64(b1), oracle.bf16_bits_to_f64(b0) * 2)


# ---- the default maths (W8A16) ------------------------------------------------
#
# * Brute force with exact rationals: Y = bf16(s_w sum x * dec(w)) with BF16
#   inputs read from their bit fields here, not through the oracle.
# * Reduction to the W8A8 chain: rows whose values are E4M3 values with a
#   largest magnitude of 448 quantise to themselves with scale 1, so both
#   definitions must give the same bits.
# * Every finite BF16 input pattern times the weight 1.0 comes back unchanged
#   (the BF16 reading of the activations and the output rounding).
# * Layout: a one-hot input row selects one column of the [out, in] weight.


def _bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite BF16 bit pattern, from its fields."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** -126
    return sign * Fraction(128 + m, 128) * Fraction(2) ** (e - 127)


def _rand_bf16(rng, shape, lo=-12, hi=6):
    """Finite BF16 patterns with exponents in [lo, hi) (both signs, zeros included)."""
    e = rng.integers(127 + lo, 127 + hi, size=shape)
    m = rng.integers(0, 128, size=shape)
    s = rng.integers(0, 2, size=shape)
    bits = (s << 15) | (e << 7) | m
    bits[rng.random(shape) < 0.05] = 0
    return bits.astype(np.uint16)


def test_w8a16_brute_force_exact_rationals():
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 40
    xb = _rand_bf16(rng, (M, K))
    qw = _rand_codes(rng, (N, K))
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    dec = {c: Fraction(float(oracle.decode(np.uint8(c)))) for c in range(256) if (c & 0x7F) != 0x7F}
    _, ybf = oracle.w8a16_linear(xb, qw, sw)
    got = oracle.bf16_bits_to_f64(ybf)
    for m in range(M):
        for n in range(N):
            acc = sum(_bf16_fraction(int(xb[m, k])) * dec[int(qw[n, k])] for k in range(K))
            want = _bf16_rne_fraction(Fraction(float(sw[n])) * acc)
            assert got[m, n] == want, (m, n)


def test_w8a16_equals_w8a8_when_quantisation_is_exact():
    rng = np.random.default_rng(12)
    M, N, K = 6, 9, 64
    codes = _rand_codes(rng, (M, K))
    codes[np.arange(M), rng.integers(0, K, M)] = 0x7E        # one element 448 per row
    x = oracle.decode(codes).astype(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)    # E4M3 values are exact in BF16
    assert np.array_equal(oracle.bf16_bits_to_f64(x_bits), oracle.decode(codes))
    q, s, _ = oracle.quantize_rows(x)
    assert np.all(s == 1.0) and np.array_equal(oracle.decode(q), oracle.decode(codes))
    qw = _rand_codes(rng, (N, K))
    sw = rng.uniform(0.01, 1, N).astype(np.float32)
    y8, b8 = oracle.w8a8_linear(q, s, qw, sw)
    y16, b16 = oracle.w8a16_linear(x_bits, qw, sw)
    assert np.array_equal(y8, y16)
    assert np.array_equal(b8, b16)


def test_w8a16_every_bf16_input_times_one():
    pats = np.arange(65536, dtype=np.uint32)
    finite = ((pats >> 7) & 0xFF) != 0xFF
    pats = pats[finite].astype(np.uint16)
    K = 16
    xb = np.zeros((pats.size, K), np.uint16)
    xb[:, 3] = pats
    qw = np.zeros((1, K), np.uint8)
    qw[0, 3] = 0x38                                           # 1.0
    y64, ybf = oracle.w8a16_linear(xb, qw, np.ones(1, np.float32))
    want = np.array([float(_bf16_fraction(int(b))) for b in pats])
    assert np.array_equal(y64[:, 0], want)
    nz = want != 0
    assert np.array_equal(ybf[nz, 0], pats[nz])               # exact values come back unchanged
    assert np.all(oracle.bf16_bits_to_f64(ybf[~nz, 0]) == 0)


def test_w8a16_one_hot_rows_select_weight_columns():
    rng = np.random.default_rng(13)
    M, N, K = 8, 12, 64
    qw = _rand_codes(rng, (N, K))
    sw = rng.uniform(0.5, 2, N).astype(np.float32)
    ks = rng.choice(K, M, replace=False)
    vals = (2.0 ** rng.integers(-3, 4, M)).astype(np.float32)
    xb = np.zeros((M, K), np.uint16)
    xb[np.arange(M), ks] = (vals.view(np.uint32) >> 16).astype(np.uint16)
    y64, _ = oracle.w8a16_linear(xb, qw, sw)
    for m in range(M):
        want = np.float64(vals[m]) * sw.astype(np.float64) * oracle.decode(qw[:, ks[m]])
        assert np.array_equal(y64[m], want)
