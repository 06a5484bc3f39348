"""Pins of the oracle's MXFP4 format, block quantiser, linear layer and
routed-expert pass.

* E2M1 decode equals the format table of the OCP MX specification
  (tests/golden/e2m1_values.txt); E8M0 decode equals torch's
  float8_e8m0fnu reading of the same bytes (library routine).
* Encoding: every value round-trips; the midpoints between neighbouring
  magnitudes go to the even mantissa and magnitudes beyond 6 saturate
  (literal cases); a brute-force nearest search over the golden table agrees
  on a dense grid.
* Block scales: for random blocks the shared exponent is the unique X with
  4 * 2**X <= amax < 8 * 2**X (searched with exact rationals), clamped to
  [-127, 127]; all-zero and tiny blocks; the largest BF16 value.
* Packing: element 2i in the low nibble (a hand-written block).
* Linear: brute force with exact rationals from the golden table, over
  several 32-blocks, so a wrong block index, nibble order or operand role
  fails.
* Routed experts: one expert at top-1 reduces to the dense MXFP4 chain;
  weight-splitting, relabelling, dropped ids and the two-pass chain act as
  they must.
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = Path(__file__).parent / "golden" / "e2m1_values.txt"


def _golden():
    table = {}
    for line in GOLDEN.read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        c, v = line.split()
        table[int(c, 16)] = float(v)
    assert len(table) == 16
    return table


def test_decode_matches_golden_table():
    table = _golden()
    got = oracle.e2m1_decode(np.arange(16))
    for c, v in table.items():
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), hex(c)


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(oracle.e8m0_value(codes), ref)


def test_encode_round_trips_every_code():
    table = _golden()
    for c, v in table.items():
        assert int(oracle.e2m1_encode(np.float64(v))) == c, hex(c)


def test_encode_ties_and_saturation():
    cases = {
        0.25: 0x0, 0.2500001: 0x1, 0.7499999: 0x1, 0.75: 0x2, 1.25: 0x2, 1.2500001: 0x3,
        1.75: 0x4, 2.5: 0x4, 2.5000001: 0x5, 3.5: 0x6, 5.0: 0x6, 5.0000001: 0x7,
        6.0: 0x7, 7.999: 0x7, 1e30: 0x7, -0.1: 0x8, -0.75: 0xA, -5.0: 0xE, -1e30: 0xF,
    }
    for v, c in cases.items():
        assert int(oracle.e2m1_encode(np.float64(v))) == c, v


def test_encode_is_nearest_over_the_table():
    table = _golden()
    pos = sorted((v, c) for c, v in table.items() if c < 8)
    grid = np.linspace(-9, 9, 14401)
    got = oracle.e2m1_encode(grid)
    for v, c in zip(grid, got):
        a = min(abs(v), 6.0)
        best = min(abs(a - m) for m, _ in pos)
        near = [cc for m, cc in pos if abs(a - m) == best]
        want = near[0] if len(near) == 1 else [cc for cc in near if cc % 2 == 0][0]
        assert (int(c) & 7) == want, v
        assert (int(c) >> 3) == (1 if np.signbit(v) else 0)


def _shared_exponent(block) -> int:
    """Brute force: the X with 4 * 2**X <= amax < 8 * 2**X, clamped to [-127, 127]."""
    amax = max(abs(Fraction(float(v))) for v in block)
    if amax == 0:
        return 0
    for X in range(-200, 200):
        if 4 * Fraction(2) ** X <= amax < 8 * Fraction(2) ** X:
            return min(max(X, -127), 127)
    raise AssertionError("no exponent")


def _encode_fraction(q: Fraction, table) -> int:
    """Nearest-even E2M1 code of an exact rational, from the golden table."""
    a = min(abs(q), Fraction(6))
    pos = sorted((Fraction(v), c) for c, v in table.items() if c < 8)
    best = min(abs(a - m) for m, _ in pos)
    near = [c for m, c in pos if abs(a - m) == best]
    c = near[0] if len(near) == 1 else [cc for cc in near if cc % 2 == 0][0]
    return c | (8 if q < 0 else 0)


def test_block_scales_and_codes_exact_rationals():
    table = _golden()
    rng = np.random.default_rng(0)
    rows = []
    for i in range(24):
        mag = 2.0 ** rng.integers(-30, 30)
        rows.append((rng.standard_normal(96) * mag).astype(np.float32))
    # amax exactly a power of two, and just below one
    rows.append(np.full(96, 2.0 ** 5, np.float32))
    rows.append(np.full(96, np.nextafter(np.float32(2.0 ** 5), np.float32(0)), np.float32))
    x = np.stack(rows)
    q, s = oracle.mx_quantize_rows(x)
    codes = oracle.mx_unpack(q)
    for r in range(x.shape[0]):
        for b in range(3):
            blk = x[r, 32 * b:32 * b + 32]
            X = _shared_exponent(blk)
            assert int(s[r, b]) == X + 127, (r, b)
            for i in range(32):
                want = _encode_fraction(Fraction(float(blk[i])) / Fraction(2) ** X, table)
                assert int(codes[r, 32 * b + i]) == want, (r, b, i)


def test_zero_tiny_and_largest_blocks():
    x = np.zeros((3, 32), np.float64)
    x[1, 3] = 2.0 ** -140            # below every scale: clamps to 2**-127, rounds to 0
    x[2, :] = -1.5
    x[2, 7] = float(bf16_bits_to_f32(np.array([0x7F7F], np.uint16))[0])  # largest BF16
    q, s = oracle.mx_quantize_rows(x)
    assert int(s[0, 0]) == 127 and not q[0].any()
    assert int(s[1, 0]) == 0 and not q[1].any()
    assert int(s[2, 0]) == 127 + 125                     # floor(log2(3.39e38)) - 2
    c = oracle.mx_unpack(q)[2]
    assert c[7] == 0x7 and c[0] == 0x8                    # -1.5 / 2**125 -> -0


def test_packing_low_nibble_first():
    x = np.zeros((1, 32))
    x[0, :4] = [1.0, -6.0, 0.5, 3.0]       # amax 6 -> X = 0, unit scale
    q, s = oracle.mx_quantize_rows(x)
    assert int(s[0, 0]) == 127
    assert list(q[0, :3]) == [0xF2, 0x51, 0x00]


def test_quantisation_error_within_half_spacing():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    q, s = oracle.mx_quantize_rows(x)
    back = oracle.mx_dequant(q, s)
    scale = np.repeat(oracle.e8m0_value(s), 32, axis=1)
    v = np.abs(x) / scale
    half = np.where(v < 2, 0.25, np.where(v < 4, 0.5, np.where(v <= 6, 1.0, 2.0)))
    assert np.all(np.abs(back - x) <= half * scale)


def _rand_mx(rng, rows, K):
    q = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    s = rng.integers(118, 137, (rows, K // 32)).astype(np.uint8)
    return q, s


def test_linear_brute_force_exact_rationals():
    table = {c: Fraction(v) for c, v in _golden().items()}
    rng = np.random.default_rng(1)
    M, N, K = 3, 4, 96
    qa, sa = _rand_mx(rng, M, K)
    qw, sw = _rand_mx(rng, N, K)
    y64, ybf = oracle.mxfp4_linear(qa, sa, qw, sw)

    def elem(q, s, r, k):
        byte = int(q[r, k // 2])
        code = byte & 0xF if k % 2 == 0 else byte >> 4
        return table[code] * Fraction(2) ** (int(s[r, k // 32]) - 127)

    for m in range(M):
        for n in range(N):
            want = sum(elem(qa, sa, m, k) * elem(qw, sw, n, k) for k in range(K))
            assert Fraction(float(y64[m, n])) == want, (m, n)
    assert np.array_equal(ybf, oracle.round_to_bf16_bits(y64))


def _small(seed=0, T=20, H=64, I=64, E=5, k=3):
    rng = np.random.default_rng(seed)
    x = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32)))
    w13 = bf16_bits_to_f32(f32_to_bf16_bits(0.05 * rng.standard_normal((E * 2 * I, H), dtype=np.float32)))
    w2 = bf16_bits_to_f32(f32_to_bf16_bits(0.05 * rng.standard_normal((E * H, I), dtype=np.float32)))
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1, (T, k)).astype(np.float32)
    q13, s13 = oracle.mx_quantize_rows(w13)
    q2, s2 = oracle.mx_quantize_rows(w2)
    return dict(x=x, ids=ids, w=w, q13=q13.reshape(E, 2 * I, H // 2), s13=s13.reshape(E, 2 * I, H // 32),
                q2=q2.reshape(E, H, I // 2), s2=s2.reshape(E, H, I // 32))


def _weights(d, inv=None):
    keys = ("q13", "s13", "q2", "s2")
    return tuple(d[k] if inv is None else d[k][inv] for k in keys)


def test_moe_single_expert_reduces_to_dense_chain():
    d = _small(E=1, k=1)
    T = d["x"].shape[0]
    ids = np.zeros((T, 1), np.int32)
    out64, out_bf, extra = oracle.moe_mxfp4_pass(d["x"], ids, np.ones((T, 1), np.float32), *_weights(d), keep=True)
    qx, sx = oracle.mx_quantize_rows(d["x"])
    gu, _ = oracle.mxfp4_linear(qx, sx, d["q13"][0], d["s13"][0])
    qh, sh = oracle.mx_quantize_rows(oracle.swiglu_f32(gu))
    y, ybf = oracle.mxfp4_linear(qh, sh, d["q2"][0], d["s2"][0])
    assert np.array_equal(extra["perm"], np.arange(T))
    assert np.array_equal(extra["qh"], qh) and np.array_equal(extra["sh"], sh)
    assert np.array_equal(out64, y) and np.array_equal(out_bf, ybf)


def test_moe_split_weights_relabelling_and_dropped_ids():
    d = _small(seed=4)
    T = d["x"].shape[0]
    base, base_bf, _ = oracle.moe_mxfp4_pass(d["x"], np.full((T, 1), 2, np.int32), np.ones((T, 1), np.float32),
                                             *_weights(d))
    out, out_bf, _ = oracle.moe_mxfp4_pass(d["x"], np.full((T, 2), 2, np.int32), np.full((T, 2), 0.5, np.float32),
                                           *_weights(d))
    assert np.array_equal(out, base) and np.array_equal(out_bf, base_bf)
    ref, _, _ = oracle.moe_mxfp4_pass(d["x"], d["ids"], d["w"], *_weights(d))
    E = d["q13"].shape[0]
    relabel = np.random.default_rng(5).permutation(E)
    inv = np.argsort(relabel)
    out2, _, _ = oracle.moe_mxfp4_pass(d["x"], relabel[d["ids"]], d["w"], *_weights(d, inv))
    assert np.array_equal(out2, ref)
    ids = d["ids"].copy()
    ids[::2, 0] = -1
    w0 = d["w"].copy()
    w0[::2, 0] = 0.0
    dropped, _, _ = oracle.moe_mxfp4_pass(d["x"], ids, d["w"], *_weights(d))
    zeroed, _, _ = oracle.moe_mxfp4_pass(d["x"], d["ids"], w0, *_weights(d))
    assert np.array_equal(dropped, zeroed)


def test_moe_combine_rounds_the_exact_sum_once():
    """Two copies of one expert with the weights 3/8 and 5/8 give the single
    copy's BF16 output; rounding each weighted copy to BF16 first would not."""
    d = _small(seed=12, T=40)
    T = d["x"].shape[0]
    base, base_bf, _ = oracle.moe_mxfp4_pass(d["x"], np.full((T, 1), 1, np.int32), np.ones((T, 1), np.float32),
                                             *_weights(d))
    w = np.tile(np.array([0.375, 0.625], np.float32), (T, 1))
    out, out_bf, _ = oracle.moe_mxfp4_pass(d["x"], np.full((T, 2), 1, np.int32), w, *_weights(d))
    assert np.allclose(out, base, rtol=2.0 ** -50, atol=0.0)
    assert np.array_equal(out_bf, base_bf)
    per_copy = oracle.round_to_bf16_bits(oracle.bf16_values(0.375 * base) + oracle.bf16_values(0.625 * base))
    assert (per_copy != base_bf).sum() > T


def test_moe_two_pass_chains_bf16_outputs():
    d = _small(seed=8)
    rng = np.random.default_rng(9)
    E, k = d["q13"].shape[0], d["ids"].shape[1]
    ids2 = np.stack([rng.choice(E, k, replace=False) for _ in range(d["x"].shape[0])]).astype(np.int32)
    routes = [(d["ids"], d["w"]), (ids2, d["w"][::-1].copy())]
    res = oracle.moe_mxfp4_two_pass(d["x"], routes, *_weights(d))
    o1, b1, _ = oracle.moe_mxfp4_pass(d["x"], *routes[0], *_weights(d))
    o2, b2, _ = oracle.moe_mxfp4_pass(bf16_bits_to_f32(b1), *routes[1], *_weights(d))
    assert np.array_equal(res[0][1], b1) and np.array_equal(res[1][1], b2)
    assert np.array_equal(res[1][0], o2)
