"""Pins of the oracle's routed-expert chain.

* Routing: the permutation is a bijection onto the valid slots, grouped by
  expert in increasing slot order; a loop-by-loop construction on small
  inputs gives the same arrays; out-of-range ids are dropped.
* One expert, top-1, weight 1 reduces to two dense layers with SwiGLU and a
  requantisation between them, computed with the dense oracle; the output
  is the second layer's BF16 output.
* k routed copies of one expert whose weights sum to 1 give that expert's
  output; relabelling experts (ids and weight stacks together) and
  reordering tokens act as they must.
* The combine rounds once: two copies of one expert with the weights 3/8
  and 5/8 give the single copy's BF16 output bit for bit, where rounding
  each weighted copy to BF16 before the sum would not (the test checks that
  the data tells the two apart).
* SiLU agrees with torch's silu in float64 (library routine).
* The two-pass stack feeds each pass the previous pass's BF16 output.
"""
import numpy as np
import torch

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits


def _small(seed=0, T=24, H=64, I=32, E=5, k=3):
    rng = np.random.default_rng(seed)
    x = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32)))
    w13 = bf16_bits_to_f32(f32_to_bf16_bits(0.05 * rng.standard_normal((E, 2 * I, H), dtype=np.float32)))
    w2 = bf16_bits_to_f32(f32_to_bf16_bits(0.05 * rng.standard_normal((E, H, I), dtype=np.float32)))
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1, (T, k)).astype(np.float32)
    qx, sx, _ = oracle.quantize_rows(x)
    q13, s13, _ = oracle.quantize_rows(w13.reshape(E * 2 * I, H))
    q2, s2, _ = oracle.quantize_rows(w2.reshape(E * H, I))
    return dict(x=x, qx=qx, sx=sx, ids=ids, w=w,
                q13=q13.reshape(E, 2 * I, H), s13=s13.reshape(E, 2 * I),
                q2=q2.reshape(E, H, I), s2=s2.reshape(E, H))


def test_route_matches_loop_construction():
    rng = np.random.default_rng(1)
    T, k, E = 50, 4, 7
    ids = rng.integers(-2, E + 2, (T, k)).astype(np.int32)
    counts, offsets, perm = oracle.route(ids, E)
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                lists[e].append(t * k + j)
    assert list(counts) == [len(l) for l in lists]
    assert list(perm) == [s for l in lists for s in l]
    assert offsets[0] == 0 and list(np.diff(offsets)) == list(counts)


def test_route_invariants_on_zipf_routing():
    from synth import routing
    ids, w = routing(np.random.default_rng(2), 512, 64, 8)
    counts, offsets, perm = oracle.route(ids, 64)
    assert counts.sum() == 512 * 8
    assert np.array_equal(np.sort(perm), np.arange(512 * 8))
    e_sorted = ids.reshape(-1)[perm]
    assert np.all(np.diff(e_sorted) >= 0)
    for e in range(64):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.allclose(w.sum(axis=1), 1, atol=1e-6)


def test_single_expert_reduces_to_dense_chain():
    d = _small(E=1, k=1)
    T = d["x"].shape[0]
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    out64, out_bf, extra = oracle.moe_pass(d["qx"], d["sx"], ids, w, d["q13"], d["s13"], d["q2"], d["s2"],
                                           keep=True)
    gu, _ = oracle.w8a8_linear(d["qx"], d["sx"], d["q13"][0], d["s13"][0])
    h = oracle.swiglu_f32(gu)
    qh, sh, _ = oracle.quantize_rows(h)
    y, ybf = oracle.w8a8_linear(qh, sh, d["q2"][0], d["s2"][0])
    assert np.array_equal(extra["perm"], np.arange(T))
    assert np.array_equal(extra["qh"], qh) and np.array_equal(extra["sh"], sh)
    assert np.array_equal(out64, y) and np.array_equal(out_bf, ybf)


def test_k_copies_of_one_expert_weights_summing_to_one():
    d = _small(E=3, k=1)
    T = d["x"].shape[0]
    ids1 = np.full((T, 1), 2, np.int32)
    base, base_bf, _ = oracle.moe_pass(d["qx"], d["sx"], ids1, np.ones((T, 1), np.float32),
                                       d["q13"], d["s13"], d["q2"], d["s2"])
    # two halves: 0.5*y + 0.5*y == y exactly in float64
    ids2 = np.full((T, 2), 2, np.int32)
    w2 = np.full((T, 2), 0.5, np.float32)
    out, out_bf, _ = oracle.moe_pass(d["qx"], d["sx"], ids2, w2, d["q13"], d["s13"], d["q2"], d["s2"])
    assert np.array_equal(out, base) and np.array_equal(out_bf, base_bf)
    # four copies with power-of-two weights: each weighted copy is an exact
    # fraction of the single copy; their float64 sum is the single copy up
    # to float64 rounding, and rounds to the same BF16
    ids4 = np.full((T, 4), 2, np.int32)
    w4 = np.tile(np.array([0.5, 0.25, 0.125, 0.125], np.float32), (T, 1))
    out4, out4_bf, _ = oracle.moe_pass(d["qx"], d["sx"], ids4, w4, d["q13"], d["s13"], d["q2"], d["s2"])
    assert np.allclose(out4, base, rtol=2.0 ** -50, atol=0.0)
    assert np.array_equal(out4_bf, base_bf)


def _per_copy_reading(copies):
    """The rejected reading of the combine, for contrast: each weighted copy
    rounded to BF16 first, then the sum rounded once more."""
    return oracle.round_to_bf16_bits(sum(oracle.bf16_values(c) for c in copies))


def test_combine_rounds_the_exact_sum_once():
    d = _small(seed=11, E=3, k=1, T=48, H=64)
    T = d["x"].shape[0]
    args = (d["q13"], d["s13"], d["q2"], d["s2"])
    base, base_bf, _ = oracle.moe_pass(d["qx"], d["sx"], np.full((T, 1), 2, np.int32), np.ones((T, 1), np.float32),
                                       *args)
    w = np.tile(np.array([0.375, 0.625], np.float32), (T, 1))
    out, out_bf, _ = oracle.moe_pass(d["qx"], d["sx"], np.full((T, 2), 2, np.int32), w, *args)
    # 3/8 y + 5/8 y is y up to float64 rounding, and y rounds to the same BF16
    assert np.allclose(out, base, rtol=2.0 ** -50, atol=0.0)
    assert np.array_equal(out_bf, base_bf)
    # the per-copy reading gives other bits on this data: the pin tells them apart
    other = _per_copy_reading([0.375 * base, 0.625 * base])
    assert (other != base_bf).sum() > T
    # three copies with weights that do not sum to a power of two: one
    # rounding of the float64 sum, taken in the order j = 0, 1, 2
    w3 = np.tile(np.array([0.3, 0.45, 0.2], np.float32), (T, 1))
    out3, out3_bf, _ = oracle.moe_pass(d["qx"], d["sx"], np.full((T, 3), 2, np.int32), w3, *args)
    wv = w3[0].astype(np.float64)
    want = (wv[0] * base + wv[1] * base) + wv[2] * base
    assert np.array_equal(out3, want)
    assert np.array_equal(out3_bf, oracle.round_to_bf16_bits(want))


def test_relabelled_experts_and_reordered_tokens():
    d = _small(seed=4)
    args = (d["q13"], d["s13"], d["q2"], d["s2"])
    out, _, _ = oracle.moe_pass(d["qx"], d["sx"], d["ids"], d["w"], *args)
    E = d["q13"].shape[0]
    relabel = np.random.default_rng(5).permutation(E)           # old id -> new id
    inv = np.argsort(relabel)                                      # new id -> old id
    out2, _, _ = oracle.moe_pass(d["qx"], d["sx"], relabel[d["ids"]], d["w"],
                                 d["q13"][inv], d["s13"][inv], d["q2"][inv], d["s2"][inv])
    # the k copies of a token are added in the same j order: identical sums
    assert np.array_equal(out2, out)
    order = np.random.default_rng(6).permutation(d["qx"].shape[0])
    out3, _, _ = oracle.moe_pass(d["qx"][order], d["sx"][order], d["ids"][order], d["w"][order], *args)
    assert np.array_equal(out3, out[order])


def test_dropped_ids_contribute_nothing():
    d = _small(seed=7)
    args = (d["q13"], d["s13"], d["q2"], d["s2"])
    ids = d["ids"].copy()
    w = d["w"].copy()
    ids[::2, 0] = -1
    out, _, _ = oracle.moe_pass(d["qx"], d["sx"], ids, w, *args)
    w0 = w.copy()
    w0[::2, 0] = 0.0
    ids0 = d["ids"].copy()
    ref, _, _ = oracle.moe_pass(d["qx"], d["sx"], ids0, w0, *args)
    assert np.array_equal(out, ref)


def test_silu_matches_torch():
    g = np.linspace(-30, 30, 10001)
    u = np.ones_like(g)
    h = oracle.swiglu_f32(np.stack([g, u], axis=1))[:, 0]
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy().astype(np.float32)
    assert np.array_equal(h, ref)
    assert oracle.swiglu_f32(np.array([[0.0, 5.0]]))[0, 0] == 0.0


def test_two_pass_chains_bf16_outputs():
    d = _small(seed=8)
    rng = np.random.default_rng(9)
    E, k = d["q13"].shape[0], d["ids"].shape[1]
    ids2 = np.stack([rng.choice(E, k, replace=False) for _ in range(d["x"].shape[0])]).astype(np.int32)
    routes = [(d["ids"], d["w"]), (ids2, d["w"][::-1].copy())]
    res = oracle.moe_two_pass(d["x"], routes, d["q13"], d["s13"], d["q2"], d["s2"])
    qx, sx, _ = oracle.quantize_rows(d["x"])
    o1, b1, _ = oracle.moe_pass(qx, sx, *routes[0], d["q13"], d["s13"], d["q2"], d["s2"])
    x2 = bf16_bits_to_f32(b1)
    qx2, sx2, _ = oracle.quantize_rows(x2)
    o2, b2, _ = oracle.moe_pass(qx2, sx2, *routes[1], d["q13"], d["s13"], d["q2"], d["s2"])
    assert np.array_equal(res[0][1], b1) and np.array_equal(res[1][1], b2)
    assert np.array_equal(res[1][0], o2)
