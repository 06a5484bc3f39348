"""GPU parity of the MXFP4 expert path against the oracle.

* mxfp4_quantize: codes and scales bit-exact (zeros, tiny, subnormal and
  largest BF16 values, exact ties, ragged K).
* Gate/up (BF16 result): every element inside the FP4 matrix-core bound.
* Fused SwiGLU + MXFP4 quantisation of h: every block scale and code
  explainable (differs from the oracle's only within the propagated error of
  a boundary), in both routing orders and across orders via dst_row.
* Down + combine fed the GPU's own h rows: every element inside the bound;
  deterministic and independent of the sorted order.
* The fused MXFP4 output quantisation equals mxfp4_quantize of the BF16
  output and the oracle's quantiser, bit for bit.
* Full pass: normalised Frobenius <= 4e-3 against the oracle, on small and
  ragged shapes, groups of 1024 rows or more (the 256 x 256 tiles, with a
  ragged N tail and half K stages), the pages' expert shapes and the two-pass
  stacks of the Praxis shape and of the 16384-token workload (pass 2
  teacher-forced); edge shapes (one token and one expert, H = I = 128,
  H = 8192, I = 2048, a zero token row) and 1024 routing groups in the
  slot-position order.
"""
import numpy as np
import pytest

import oracle
from gpu_util import bf16_bits, record, to_dev, to_dev_bf16
from moe_util import bf16_compare
from mx_util import check_mx_requant, down_combine_ref, quantized_mx_moe, sorted_rows_gate_up

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import w8a8_fp8_linear_amd as w8  # noqa: E402

SMALL = dict(T=37, H=256, I=256, E=5, k=3, n_outlier=2)
RAGGED = dict(T=301, H=384, I=384, E=9, k=4, n_outlier=3)   # a half K stage, 3 gate/up tiles, odd groups
MID = dict(T=960, H=384, I=384, E=4, k=2, n_outlier=3)       # 480 rows per group: the 128 x 128 tiles
PRAXIS = dict(T=4096, H=1024, I=512, E=128, k=4, n_outlier=10, passes=2)


@pytest.fixture(scope="module")
def small():
    d = quantized_mx_moe(**SMALL, seed=5)
    ids, w = d["routes"][0]
    ids = ids.copy()
    ids[3, 1] = -1
    ids[10, 0] = SMALL["E"]
    d["routes"][0] = (ids, w)
    return d


@pytest.fixture(scope="module")
def ragged():
    return quantized_mx_moe(**RAGGED, seed=11)


@pytest.fixture(scope="module")
def mid():
    return quantized_mx_moe(**MID, seed=13)


@pytest.fixture(scope="module")
def praxis():
    return quantized_mx_moe(**PRAXIS, seed=0)


def _dev(d):
    return {k: to_dev(d[k]) for k in ("qx", "sx", "q13", "s13", "q2", "s2")}


def _slot_position_ids(ids, E):
    ids = np.asarray(ids)
    j = np.arange(ids.shape[1])[None, :]
    return np.where((ids >= 0) & (ids < E), j * E + ids, -1).astype(np.int32)


def _oracle_route(ids, E, order):
    if order == 0:
        return oracle.route(ids, E)
    return oracle.route(_slot_position_ids(ids, E), ids.shape[1] * E)


# ---- quantiser ------------------------------------------------------------------

def _special_rows(K):
    rng = np.random.default_rng(7)
    rows = []
    rows.append(np.zeros(K, np.float32))
    r = np.zeros(K, np.float32)
    r[5 % K] = -0.0
    r[40 % K] = 2.0 ** -133                      # smallest BF16 subnormal
    r[70 % K] = 1e-39                            # a BF16 subnormal block maximum
    rows.append(r)
    big = rng.standard_normal(K).astype(np.float32)
    big[::32] = 3.3895313892515355e38             # largest BF16
    rows.append(big)
    ties = np.tile(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32), K // 8)
    rows.append(ties)                            # amax 6 -> unit scale: every tie rounds to even
    rows.append(-ties * 2.0 ** -100)
    rows.append((rng.standard_normal(K) * np.exp2(rng.integers(-60, 60, K))).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (300, 2080), (64, 4096)])
def test_mxfp4_quantize_bitexact(M, K):
    print(f"[mx quantize] M={M} K={K}", flush=True)
    rng = np.random.default_rng(M + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 20, (M, K // 32)).repeat(32, axis=1)))
    x = np.concatenate([_special_rows(K), x.astype(np.float32)])
    bits = oracle.round_to_bf16_bits(x)
    x32 = oracle.bf16_bits_to_f64(bits).astype(np.float32)
    q, s = w8.mxfp4_quantize(to_dev_bf16(bits))
    torch.cuda.synchronize()
    qo, so = oracle.mx_quantize_rows(x32)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


def test_mxfp4_quantize_workload_rows():
    """The token rows of the Praxis-shaped workload (4096 x 1024, outlier channels)."""
    d = quantized_mx_moe(T=4096, H=1024, I=128, E=1, k=1, n_outlier=10, seed=3)
    q, s = w8.mxfp4_quantize(to_dev_bf16(d["x_bits"]))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), d["sx"]) and np.array_equal(q.cpu().numpy(), d["qx"])


# ---- gate/up ----------------------------------------------------------------------

def _check_gate_up_bf16(d, order=0):
    dv = _dev(d)
    ids, _ = d["routes"][0]
    _, offsets, perm = w8.moe_route(to_dev(ids), d["E"], order=order)
    gu = w8.moe_mxfp4_gate_up_bf16(dv["qx"], dv["sx"], perm, offsets, dv["q13"], dv["s13"], d["k"], order=order)
    torch.cuda.synchronize()
    _, ro, rp = _oracle_route(ids, d["E"], order)
    assert np.array_equal(perm.cpu().numpy()[:rp.size], rp)
    gu64, err = sorted_rows_gate_up(d["qx"], d["sx"], ids, rp, np.arange(rp.size), d["q13"], d["s13"], d["k"])
    rep = bf16_compare(bf16_bits(gu)[:rp.size], gu64, err)
    print("mx gate/up bf16", rep, flush=True)
    record(f"mxfp4 gate/up bf16 T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']} order={order}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep


@pytest.mark.parametrize("order", [0, 1])
def test_gate_up_bf16_small(small, order):
    _check_gate_up_bf16(small, order)


def test_gate_up_bf16_ragged(ragged):
    _check_gate_up_bf16(ragged)


def test_gate_up_bf16_mid(mid):
    _check_gate_up_bf16(mid)


def _check_fused(d, tile_order=0, row_order=0, sample=None):
    dv = _dev(d)
    ids, _ = d["routes"][0]
    ids_dev = to_dev(ids)
    _, off_r, perm_r, row_r = w8.moe_route(ids_dev, d["E"], order=row_order, with_slot_row=True)
    if tile_order == row_order:
        perm_t, off_t, dst = perm_r, off_r, None
    else:
        _, off_t, perm_t = w8.moe_route(ids_dev, d["E"], order=tile_order)
        dst = row_r
    hq, hs = w8.moe_mxfp4_gate_up_swiglu_quant(dv["qx"], dv["sx"], perm_t, off_t, dv["q13"], dv["s13"], d["k"],
                                               order=tile_order, dst_row=dst)
    torch.cuda.synchronize()
    _, _, rp = _oracle_route(ids, d["E"], row_order)
    assert np.array_equal(perm_r.cpu().numpy()[:rp.size], rp)
    rows = np.arange(rp.size) if sample is None else np.sort(
        np.random.default_rng(1).choice(rp.size, min(sample, rp.size), replace=False))
    gu64, err = sorted_rows_gate_up(d["qx"], d["sx"], ids, rp, rows, d["q13"], d["s13"], d["k"])
    rep = check_mx_requant(hq.cpu().numpy()[rows], hs.cpu().numpy()[rows], gu64, err)
    print("mx fused swiglu+quant", rep, flush=True)
    record(f"mxfp4 fused swiglu+quant T={d['T']} I={d['I']} E={d['E']} k={d['k']} tiles=order{tile_order} "
           f"rows=order{row_order} n={len(rows)}", rep)
    return hq, hs, perm_r, off_r


@pytest.mark.parametrize("tile_order,row_order", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_fused_quant_small(small, tile_order, row_order):
    _check_fused(small, tile_order, row_order)


def test_fused_quant_ragged(ragged):
    _check_fused(ragged)


def test_fused_quant_mid(mid):
    _check_fused(mid)


# ---- down + combine ---------------------------------------------------------------

def _check_down(d, hq, hs, perm, offsets, order=0, n_tokens=None, route_idx=0):
    dv = _dev(d)
    ids, tw = d["routes"][route_idx]
    out = w8.moe_mxfp4_down_combine(hq, hs, perm, offsets, to_dev(ids), to_dev(tw), dv["q2"], dv["s2"], order=order)
    torch.cuda.synchronize()
    tokens = np.arange(d["T"]) if n_tokens is None else np.sort(
        np.random.default_rng(2).choice(d["T"], n_tokens, replace=False))
    ref64, err = down_combine_ref(hq.cpu().numpy(), hs.cpu().numpy(), perm.cpu().numpy(), ids, tw, d["q2"], d["s2"],
                                  d["k"], tokens)
    rep = bf16_compare(bf16_bits(out)[tokens], ref64, err)
    print("mx down+combine", rep, flush=True)
    record(f"mxfp4 down+combine T={d['T']} H={d['H']} order={order} tokens={len(tokens)}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep
    return out


@pytest.mark.parametrize("order", [0, 1])
def test_down_combine_small(small, order):
    hq, hs, perm, offsets = _check_fused(small, order, order)
    _check_down(small, hq, hs, perm, offsets, order=order)


def test_down_combine_ragged(ragged):
    hq, hs, perm, offsets = _check_fused(ragged)
    _check_down(ragged, hq, hs, perm, offsets)


def test_down_combine_mid(mid):
    hq, hs, perm, offsets = _check_fused(mid)
    _check_down(mid, hq, hs, perm, offsets)


def test_down_combine_deterministic_and_order_independent(small):
    ids, tw = small["routes"][0]
    dv = _dev(small)
    outs = []
    for order in (0, 1, 0):
        hq, hs, perm, offsets = _check_fused(small, order, order)
        outs.append(bf16_bits(w8.moe_mxfp4_down_combine(hq, hs, perm, offsets, to_dev(ids), to_dev(tw), dv["q2"],
                                                        dv["s2"], order=order)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ---- full pass -------------------------------------------------------------------

def _oracle_tokens(x32, ids, w, d, tokens):
    out64, _, _ = oracle.moe_mxfp4_pass(x32[tokens], ids[tokens], w[tokens], d["q13"], d["s13"], d["q2"], d["s2"])
    return out64


def _check_full_pass_stagewise(d, out):
    """The full pass equals the stage-by-stage chain bit for bit, and each
    stage of that chain is checked element by element on every slot and token
    (the fused h quantisation by the explainable rule, the down projection +
    combine inside the element bound)."""
    hq, hs, perm, offsets = _check_fused(d)
    chain = _check_down(d, hq, hs, perm, offsets)
    assert np.array_equal(bf16_bits(chain), bf16_bits(out)), "the full pass differs from the stage-by-stage chain"


@pytest.mark.parametrize("cfg", ["small", "ragged", "mid"])
def test_full_pass(cfg, request):
    d = request.getfixturevalue(cfg)
    dv = _dev(d)
    ids, w = d["routes"][0]
    out = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    _check_full_pass_stagewise(d, out)
    rep = bf16_compare(bf16_bits(out), _oracle_tokens(d["x32"], ids, w, d, np.arange(d["T"])))
    print(f"mx full pass {cfg}", rep, flush=True)
    record(f"mxfp4 full pass {cfg} T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']}", rep)
    assert rep["frobenius"] <= 4e-3, rep


@pytest.mark.parametrize("cfg", [dict(T=37, H=256, I=256, E=5, k=3), dict(T=301, H=384, I=384, E=9, k=4),
                                 dict(T=64, H=2176, I=128, E=4, k=2)])
def test_fused_output_quantisation(cfg):
    print(f"[mx fused out quant] {cfg}", flush=True)
    d = quantized_mx_moe(**cfg, n_outlier=2, seed=17)
    dv = _dev(d)
    ids, w = d["routes"][0]
    args = (dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    plain = w8.moe_mxfp4_grouped(*args)
    out, q, s = w8.moe_mxfp4_grouped(*args, quantize_output=True)
    q2, s2 = w8.mxfp4_quantize(out)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), bf16_bits(plain))
    assert np.array_equal(q.cpu().numpy(), q2.cpu().numpy()) and np.array_equal(s.cpu().numpy(), s2.cpu().numpy())
    qo, so = oracle.mx_quantize_rows(oracle.bf16_bits_to_f64(bf16_bits(out)).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)


@pytest.mark.parametrize("E", [128, 192])
def test_pages_expert_shapes(E):
    """128 or 192 experts, latent width 1024, top-4 (intermediate width 512 is a
    reading): a full pass on 512 tokens, checked stage by stage and end to end
    against the oracle on every token."""
    print(f"[mx pages shape] E={E}", flush=True)
    d = quantized_mx_moe(T=512, H=1024, I=512, E=E, k=4, n_outlier=5, seed=E)
    dv = _dev(d)
    ids, w = d["routes"][0]
    out = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    _check_full_pass_stagewise(d, out)
    rep = bf16_compare(bf16_bits(out), _oracle_tokens(d["x32"], ids, w, d, np.arange(d["T"])))
    print(f"mx pages shape E={E}", rep, flush=True)
    record(f"mxfp4 full pass pages shape T=512 H=1024 I=512 E={E} k=4", rep)
    assert rep["frobenius"] <= 4e-3, rep


def test_two_pass_praxis(praxis):
    """The Praxis-shaped prefill workload (4096 tokens, 128 experts, top-4), two
    passes on one set of weights; 256 sampled tokens per pass, pass 2
    teacher-forced from the GPU's pass-1 output. Fused stages checked on
    sampled rows."""
    d = praxis
    dv = _dev(d)
    hq, hs, perm, offsets = _check_fused(d, sample=2048)
    _check_down(d, hq, hs, perm, offsets, n_tokens=256)
    routes_dev = [(to_dev(i), to_dev(w)) for i, w in d["routes"]]
    ws = w8.moe_mxfp4_workspace(d["T"], d["H"], d["I"], d["E"], d["k"])
    outs = w8.moe_mxfp4_ffn(to_dev_bf16(d["x_bits"]), routes_dev, dv["q13"], dv["s13"], dv["q2"], dv["s2"],
                            workspace=ws)
    torch.cuda.synchronize()
    tokens = np.sort(np.random.default_rng(3).choice(d["T"], 256, replace=False))
    ids1, w1 = d["routes"][0]
    rep1 = bf16_compare(bf16_bits(outs[0])[tokens], _oracle_tokens(d["x32"], ids1, w1, d, tokens))
    print("mx pass 1", rep1, flush=True)
    record("mxfp4 two-pass Praxis shape T=4096 pass 1 (256 tokens)", rep1)
    assert rep1["frobenius"] <= 4e-3, rep1
    x2 = oracle.bf16_bits_to_f64(bf16_bits(outs[0])[tokens]).astype(np.float32)
    ids2, w2 = d["routes"][1]
    ref2, _, _ = oracle.moe_mxfp4_pass(x2, ids2[tokens], w2[tokens], d["q13"], d["s13"], d["q2"], d["s2"])
    rep2 = bf16_compare(bf16_bits(outs[1])[tokens], ref2)
    print("mx pass 2 (teacher-forced)", rep2, flush=True)
    record("mxfp4 two-pass Praxis shape T=4096 pass 2 teacher-forced (256 tokens)", rep2)
    assert rep2["frobenius"] <= 4e-3, rep2


# Groups of 1024 rows or more on average run the 256 x 256 tiles (smaller
# averages run 128 x 128 or 64 x 128 tiles): the shapes the 16384-token
# workload reaches, plus a ragged N tail, half K stages and one n-tile.
MX_LARGE_TILE_MIN_ROWS = 1024
MX_LARGE_GROUPS = [
    dict(T=2200, H=2176, I=384, E=2, k=1, n_outlier=3),   # N tail 2176 = 8 x 256 + 128; K 8.5 and 1.5 stages
    dict(T=1100, H=256, I=1280, E=1, k=1, n_outlier=2),   # 5 K stages in the down projection, one n-tile
    dict(T=4096, H=2048, I=512, E=2, k=2, n_outlier=4),   # the workload's H and I; more tiles than CUs
]


@pytest.mark.parametrize("cfg", MX_LARGE_GROUPS)
@pytest.mark.parametrize("order", [0, 1])
def test_large_groups(cfg, order):
    print(f"[mx large groups] {cfg} order={order}", flush=True)
    groups = cfg["E"] * (cfg["k"] if order else 1)
    assert cfg["T"] * cfg["k"] // groups >= MX_LARGE_TILE_MIN_ROWS
    d = quantized_mx_moe(**cfg, seed=23)
    hq, hs, perm, offsets = _check_fused(d, order, order, sample=2048)
    chain = _check_down(d, hq, hs, perm, offsets, order=order, n_tokens=min(512, d["T"]))
    if order == 0:
        _check_gate_up_bf16(d)
        dv = _dev(d)
        ids, w = d["routes"][0]
        out = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"],
                                   dv["s2"])
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(chain), bf16_bits(out)), "the full pass differs from the stage chain"
        tokens = np.sort(np.random.default_rng(5).choice(d["T"], min(256, d["T"]), replace=False))
        rep = bf16_compare(bf16_bits(out)[tokens], _oracle_tokens(d["x32"], ids, w, d, tokens))
        record(f"mxfp4 full pass large groups T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']}", rep)
        assert rep["frobenius"] <= 4e-3, rep


def test_two_pass_workload_sampled():
    """The 16384-token MXFP4 two-pass workload (H 2048, I 512, 64 experts,
    top-8: about 2048 rows per group, the 256 x 256 tiles), as the benchmark
    runs it: the fused stages on sampled rows and tokens, then both passes end
    to end on 256 sampled tokens, pass 2 from the GPU's pass-1 output."""
    d = quantized_mx_moe(T=16384, H=2048, I=512, E=64, k=8, n_outlier=20, passes=2, seed=0)
    dv = _dev(d)
    hq, hs, perm, offsets = _check_fused(d, sample=2048)
    _check_down(d, hq, hs, perm, offsets, n_tokens=256)
    routes_dev = [(to_dev(i), to_dev(w)) for i, w in d["routes"]]
    ws = w8.moe_mxfp4_workspace(d["T"], d["H"], d["I"], d["E"], d["k"])
    outs = w8.moe_mxfp4_ffn(to_dev_bf16(d["x_bits"]), routes_dev, dv["q13"], dv["s13"], dv["q2"], dv["s2"],
                            workspace=ws)
    torch.cuda.synchronize()
    tokens = np.sort(np.random.default_rng(6).choice(d["T"], 256, replace=False))
    ids1, w1 = d["routes"][0]
    rep1 = bf16_compare(bf16_bits(outs[0])[tokens], _oracle_tokens(d["x32"], ids1, w1, d, tokens))
    print("mx workload pass 1", rep1, flush=True)
    record("mxfp4 two-pass T=16384 pass 1 (256 tokens)", rep1)
    assert rep1["frobenius"] <= 4e-3, rep1
    x2 = oracle.bf16_bits_to_f64(bf16_bits(outs[0])[tokens]).astype(np.float32)
    ids2, w2 = d["routes"][1]
    ref2, _, _ = oracle.moe_mxfp4_pass(x2, ids2[tokens], w2[tokens], d["q13"], d["s13"], d["q2"], d["s2"])
    rep2 = bf16_compare(bf16_bits(outs[1])[tokens], ref2)
    print("mx workload pass 2 (teacher-forced)", rep2, flush=True)
    record("mxfp4 two-pass T=16384 pass 2 teacher-forced (256 tokens)", rep2)
    assert rep2["frobenius"] <= 4e-3, rep2


def test_all_slots_dropped_gives_zeros(small):
    dv = _dev(small)
    T, k = small["T"], small["k"]
    ids = np.full((T, k), -1, np.int32)
    out = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(np.ones((T, k), np.float32)), dv["q13"],
                               dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    assert not bf16_bits(out).any()


def test_partly_dropped_slots(ragged):
    """Some slots dropped (id -1, or an id outside [0, E)): the full pass against
    the oracle on every token and against the stage chain bit for bit; a token
    with no valid slot left comes out zero."""
    d = dict(ragged)
    ids, w = d["routes"][0]
    ids = ids.copy()
    ids[::3, 0] = -1
    ids[1::5, -1] = d["E"] + 2
    ids[7] = -1
    d["routes"] = [(ids, w)] + list(d["routes"][1:])
    dv = _dev(d)
    out = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    _check_full_pass_stagewise(d, out)
    rep = bf16_compare(bf16_bits(out), _oracle_tokens(d["x32"], ids, w, d, np.arange(d["T"])))
    assert rep["frobenius"] <= 4e-3, rep
    assert not bf16_bits(out)[7].any()


@pytest.mark.parametrize("cfg", [dict(T=1, H=128, I=128, E=1, k=1), dict(T=3, H=128, I=128, E=2, k=2),
                                 dict(T=70, H=8192, I=128, E=3, k=2), dict(T=40, H=128, I=2048, E=4, k=3)])
def test_edge_shapes_full_pass(cfg):
    """One token and one expert; the smallest sizes (H = I = 128); a wide latent
    (H = 8192: 32 K steps in the gate/up, 32 output tiles in the down
    projection); a wide intermediate (I = 2048). A zero token row is included
    where there is more than one token. Full pass against the oracle, and the
    fused MXFP4 output quantisation bit-exact against the oracle's quantiser."""
    print(f"[mx edge] {cfg}", flush=True)
    d = quantized_mx_moe(**cfg, n_outlier=1, seed=31)
    if cfg["T"] > 1:
        d["x_bits"] = d["x_bits"].copy()
        d["x_bits"][0] = 0
        d["x32"] = oracle.bf16_bits_to_f64(d["x_bits"]).astype(np.float32)
        d["qx"], d["sx"] = oracle.mx_quantize_rows(d["x32"])
    dv = _dev(d)
    ids, w = d["routes"][0]
    out, q, s = w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"],
                                     dv["s2"], quantize_output=True)
    torch.cuda.synchronize()
    got = bf16_bits(out)
    rep = bf16_compare(got, _oracle_tokens(d["x32"], ids, w, d, np.arange(d["T"])))
    record(f"mxfp4 edge shape T={cfg['T']} H={cfg['H']} I={cfg['I']} E={cfg['E']} k={cfg['k']}", rep)
    assert rep["frobenius"] <= 4e-3, rep
    if cfg["T"] > 1:
        assert not got[0].any()
    qo, so = oracle.mx_quantize_rows(oracle.bf16_bits_to_f64(got).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(s.cpu().numpy(), so)


def test_slot_position_order_with_1024_groups():
    """Order 1 with top-16 of 64 experts: 1024 routing groups, most of them tiny,
    through the fused gate/up and the down projection."""
    d = quantized_mx_moe(T=200, H=256, I=128, E=64, k=16, n_outlier=1, seed=37)
    hq, hs, perm, offsets = _check_fused(d, tile_order=1, row_order=1)
    _check_down(d, hq, hs, perm, offsets, order=1)


def test_mxfp4_argument_errors(small):
    dv = _dev(small)
    T, k = small["T"], small["k"]
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.ones((T, k), dtype=torch.float32, device="cuda")
    E, H = small["E"], small["H"]
    q13 = torch.zeros((E, 2 * 96, H // 2), dtype=torch.uint8, device="cuda")   # I = 96: not a multiple of 128
    s13 = torch.zeros((E, 2 * 96, H // 32), dtype=torch.uint8, device="cuda")
    q2 = torch.zeros((E, H, 48), dtype=torch.uint8, device="cuda")
    s2 = torch.zeros((E, H, 3), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # the binding finds no workspace size for I = 96
        w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], ids, w, q13, s13, q2, s2)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:      # and the library refuses it
        w8.moe_mxfp4_grouped(dv["qx"], dv["sx"], ids, w, q13, s13, q2, s2, workspace=ws)
    assert e.value.status == 4
    with pytest.raises(ValueError):   # scales that do not match the codes
        w8.moe_mxfp4_grouped(dv["qx"], dv["sx"][:, :-1].contiguous(), ids, w, dv["q13"], dv["s13"], dv["q2"],
                             dv["s2"])
    with pytest.raises(w8.W8A8Error) as e:
        w8.mxfp4_quantize(torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda"))   # K % 32
    assert e.value.status == 4
