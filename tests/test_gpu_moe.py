"""GPU parity of the routed-expert path against the oracle.

* moe_route: counts, offsets and the permutation are bit-exact.
* Gate/up (BF16 result): every element inside the E4M3 matrix-core bound.
* Fused SwiGLU + requantisation: scales within the propagated bound and
  every code explainable (differs from the oracle's only where the oracle's
  scaled value lies within the propagated error of a rounding boundary).
* The requantisation on the GPU's own float32 h rows: codes and scales equal
  the oracle's quantiser bit for bit (small shapes, the 4096-token workload,
  a 256 x 256-tile shape), and h within its propagated bound.
* Down + combine: fed the GPU's own requantised rows, every output element
  of the sampled tokens inside the bound (the weighted copies summed at full
  precision and rounded once).
* Full pass: normalised Frobenius <= 4e-3 against the oracle. The two-pass
  stack: the benched entry point equals the stage-by-stage chain bit for
  bit, every stage is checked element by element on its own GPU input, and
  each pass end to end within Frobenius 4e-3 (pass 2 from the GPU's pass-1
  output).
Shapes: the routed-expert workloads (4096 and 16384 tokens, H 2048, I 512,
64 experts, top-8, Zipf routing) and small ragged ones.
"""
import numpy as np
import pytest

import oracle
from gpu_util import bf16_bits, record, to_dev
from moe_util import (bf16_compare, check_requant, down_combine_ref, quantized_moe,
                      sorted_rows_gate_up, swiglu_bound)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import w8a8_fp8_linear_amd as w8  # noqa: E402

SMALL = dict(T=37, H=256, I=256, E=5, k=3, n_outlier=2)
RAGGED = dict(T=301, H=272, I=384, E=9, k=4, n_outlier=3)   # K tail, 3 gate/up tiles, odd groups
MID = dict(T=500, H=272, I=384, E=4, k=2, n_outlier=3)       # 250 rows per group: the 128 x 128 tiles
GATE_UP = dict(T=4096, H=2048, I=512, E=64, k=8, n_outlier=20)
TWO_PASS = dict(T=16384, H=2048, I=512, E=64, k=8, n_outlier=20, passes=2)


@pytest.fixture(scope="module")
def small():
    d = quantized_moe(**SMALL, seed=5)
    ids, w = d["routes"][0]
    ids = ids.copy()
    ids[3, 1] = -1          # dropped slots
    ids[10, 0] = SMALL["E"]
    d["routes"][0] = (ids, w)
    return d


@pytest.fixture(scope="module")
def ragged():
    return quantized_moe(**RAGGED, seed=11)


@pytest.fixture(scope="module")
def mid():
    return quantized_moe(**MID, seed=13)


@pytest.fixture(scope="module")
def gate_up_cfg():
    return quantized_moe(**GATE_UP, seed=0)


@pytest.fixture(scope="module")
def two_pass_cfg():
    return quantized_moe(**TWO_PASS, seed=0)


def _dev(d):
    return {"qx": to_dev(d["qx"]), "sx": to_dev(d["sx"]), "q13": to_dev(d["q13"]), "s13": to_dev(d["s13"]),
            "q2": to_dev(d["q2"]), "s2": to_dev(d["s2"])}


def slot_position_ids(ids, E):
    """Group keys of the slot-position-major order: j * E + e (invalid ids stay invalid)."""
    ids = np.asarray(ids)
    j = np.arange(ids.shape[1])[None, :]
    return np.where((ids >= 0) & (ids < E), j * E + ids, -1).astype(np.int32)


def oracle_route(ids, E, order):
    if order == 0:
        return oracle.route(ids, E)
    return oracle.route(slot_position_ids(ids, E), ids.shape[1] * E)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (37, 3, 5), (1000, 8, 7), (4096, 8, 64), (16384, 8, 64),
                                   (513, 4, 130), (2000, 2, 1024), (300, 64, 16)])
def test_route_bitexact(T, k, E, order):
    if order == 1 and k * E > 1024:
        pytest.skip("more than 1024 routing groups")
    print(f"[route] T={T} k={k} E={E} order={order}", flush=True)
    rng = np.random.default_rng(T + k + E)
    ids = rng.integers(-1, E + 1, (T, k)).astype(np.int32)
    if E == 64:
        from synth import routing
        ids, _ = routing(rng, T, E, k)
    counts, offsets, perm, slot_row = w8.moe_route(to_dev(ids), E, order, with_slot_row=True)
    torch.cuda.synchronize()
    rc, ro, rp = oracle_route(ids, E, order)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    p = perm.cpu().numpy()
    assert np.array_equal(p[:rp.size], rp)
    assert np.all(p[rp.size:] == -1)
    # slot_row is the inverse permutation, -1 on dropped slots
    want = np.full(T * k, -1, np.int64)
    want[rp] = np.arange(rp.size)
    assert np.array_equal(slot_row.cpu().numpy(), want)


def test_route_deterministic():
    from synth import routing
    ids, _ = routing(np.random.default_rng(1), 4096, 64, 8)
    a = w8.moe_route(to_dev(ids), 64)[2].cpu().numpy()
    b = w8.moe_route(to_dev(ids), 64)[2].cpu().numpy()
    assert np.array_equal(a, b)


def _check_gate_up_bf16(d, sample=None):
    dv = _dev(d)
    ids, _ = d["routes"][0]
    gu, perm, offsets = w8.w8a8_grouped_gemm(dv["qx"], dv["sx"], to_dev(ids), dv["q13"], dv["s13"])
    torch.cuda.synchronize()
    _, ro, rp = oracle.route(ids, d["E"])
    assert np.array_equal(perm.cpu().numpy()[:rp.size], rp)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    rows = np.arange(rp.size) if sample is None else np.sort(
        np.random.default_rng(0).choice(rp.size, min(sample, rp.size), replace=False))
    gu64, err = sorted_rows_gate_up(d["qx"], d["sx"], ids, rp, rows, d["q13"], d["s13"], d["k"])
    got = bf16_bits(gu)[rows]
    rep = bf16_compare(got, gu64, err)
    print("gate/up bf16", rep, flush=True)
    record(f"moe gate/up bf16 T={d['T']} E={d['E']} k={d['k']}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep


def test_gate_up_bf16_small(small):
    _check_gate_up_bf16(small)


def test_gate_up_bf16_mid(mid):
    """Groups of about 250 rows (the 128 x 128 tile shape)."""
    _check_gate_up_bf16(mid)


def test_gate_up_bf16_full_size(gate_up_cfg):
    """4096 tokens, top-8 of 64 experts, [1024 x 2048] gate+up per expert: every row."""
    _check_gate_up_bf16(gate_up_cfg)


def _check_fused_requant(d, route_idx=0, sample=None, tile_order=0, row_order=0):
    """Fused gate/up + SwiGLU + requantisation with tiles in `tile_order` and
    h rows in `row_order` (different orders go through dst_row = the
    row order's slot_row). Returns (h_q, h_scale, perm, offsets) of the row
    order."""
    dv = _dev(d)
    ids, _ = d["routes"][route_idx]
    ids_dev = to_dev(ids)
    _, off_r, perm_r, row_r = w8.moe_route(ids_dev, d["E"], order=row_order, with_slot_row=True)
    if tile_order == row_order:
        perm_t, off_t, dst = perm_r, off_r, None
    else:
        _, off_t, perm_t = w8.moe_route(ids_dev, d["E"], order=tile_order)
        dst = row_r
    hq, hs = w8.moe_gate_up_swiglu_quant(dv["qx"], dv["sx"], perm_t, off_t, dv["q13"], dv["s13"], d["k"],
                                         order=tile_order, dst_row=dst)
    torch.cuda.synchronize()
    _, _, rp = oracle_route(ids, d["E"], row_order)
    assert np.array_equal(perm_r.cpu().numpy()[:rp.size], rp)
    rows = np.arange(rp.size) if sample is None else np.sort(
        np.random.default_rng(1).choice(rp.size, min(sample, rp.size), replace=False))
    gu64, err = sorted_rows_gate_up(d["qx"], d["sx"], ids, rp, rows, d["q13"], d["s13"], d["k"])
    rep = check_requant(hq.cpu().numpy()[rows], hs.cpu().numpy()[rows], gu64, err)
    print("fused requant", rep, flush=True)
    record(f"moe fused swiglu+requant T={d['T']} E={d['E']} k={d['k']} I={d['I']} tiles=order{tile_order} "
           f"rows=order{row_order} n={len(rows)}", rep)
    return hq, hs, perm_r, off_r


@pytest.mark.parametrize("tile_order,row_order", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_fused_requant_small(small, tile_order, row_order):
    _check_fused_requant(small, tile_order=tile_order, row_order=row_order)


@pytest.mark.parametrize("tile_order,row_order", [(0, 0), (1, 1), (0, 1)])
def test_fused_requant_ragged(ragged, tile_order, row_order):
    """I = 384 (three 128-column h tiles), H = 272 (a 16-byte K tail), 9 experts."""
    _check_fused_requant(ragged, tile_order=tile_order, row_order=row_order)


def test_fused_requant_mid(mid):
    _check_fused_requant(mid)


def test_fused_requant_gate_up_cfg(gate_up_cfg):
    _check_fused_requant(gate_up_cfg, sample=4096)


def _check_down(d, hq, hs, perm, offsets, route_idx=0, n_tokens=None, order=0):
    dv = _dev(d)
    ids, tw = d["routes"][route_idx]
    out = w8.moe_down_combine(hq, hs, perm, offsets, to_dev(ids), to_dev(tw), dv["q2"], dv["s2"], order=order)
    torch.cuda.synchronize()
    T = d["T"]
    tokens = np.arange(T) if n_tokens is None else np.sort(
        np.random.default_rng(2).choice(T, n_tokens, replace=False))
    ref64, err = down_combine_ref(hq.cpu().numpy(), hs.cpu().numpy(), perm.cpu().numpy(), ids, tw,
                                  d["q2"], d["s2"], d["k"], tokens)
    rep = bf16_compare(bf16_bits(out)[tokens], ref64, err)
    print("down+combine", rep, flush=True)
    record(f"moe down+combine T={d['T']} order={order} tokens={len(tokens)}", rep)
    assert rep["n_bound_violations"] == 0, rep
    assert rep["frobenius"] <= 4e-3, rep


@pytest.mark.parametrize("order", [0, 1])
def test_down_combine_small(small, order):
    hq, hs, perm, offsets = _check_fused_requant(small, tile_order=order, row_order=order)
    _check_down(small, hq, hs, perm, offsets, order=order)


def test_down_combine_ragged(ragged):
    hq, hs, perm, offsets = _check_fused_requant(ragged)
    _check_down(ragged, hq, hs, perm, offsets)


def test_down_combine_mid(mid):
    hq, hs, perm, offsets = _check_fused_requant(mid)
    _check_down(mid, hq, hs, perm, offsets)


# Groups of 1024 rows or more on average: the 256 x 256 tiles (smaller
# averages run 128 x 128 or 64 x 128 tiles), on shapes the workloads above
# do not reach: a ragged N tail, 6 and 8 K steps in the down projection, one
# n-tile, more tiles than CUs.
LARGE_TILE_MIN_ROWS = 1024
LARGE_GROUPS = [
    dict(T=2200, H=2064, I=512, E=2, k=1, n_outlier=3),   # an N tail: 2064 = 8 x 256 + 16
    dict(T=1100, H=512, I=1024, E=1, k=1, n_outlier=2),   # 8 K steps
    dict(T=1100, H=256, I=768, E=1, k=1, n_outlier=2),    # 6 K steps, one n-tile
    dict(T=4096, H=2048, I=512, E=2, k=2, n_outlier=4),   # 272 tiles: more than one per workgroup
]


@pytest.mark.parametrize("cfg", LARGE_GROUPS)
@pytest.mark.parametrize("order", [0, 1])
def test_down_combine_large_groups(cfg, order):
    print(f"[large groups] {cfg} order={order}", flush=True)
    groups = cfg["E"] * (cfg["k"] if order else 1)
    assert cfg["T"] * cfg["k"] // groups >= LARGE_TILE_MIN_ROWS
    d = quantized_moe(**cfg, seed=17)
    hq, hs, perm, offsets = _check_fused_requant(d, tile_order=order, row_order=order, sample=2048)
    _check_down(d, hq, hs, perm, offsets, n_tokens=min(512, d["T"]), order=order)


def _check_requant_bitexact(d, route_idx=0, sample=None):
    """The fused gate/up + SwiGLU + requantisation, with the float32 h rows the
    codes were made from: the codes and scales must equal the oracle's
    quantiser on those h rows bit for bit, and h itself must lie within the
    bound carried from the gate/up products."""
    dv = _dev(d)
    ids, _ = d["routes"][route_idx]
    _, off, perm = w8.moe_route(to_dev(ids), d["E"])
    hq, hs, h = w8.moe_gate_up_swiglu_quant(dv["qx"], dv["sx"], perm, off, dv["q13"], dv["s13"], d["k"],
                                            return_h=True)
    torch.cuda.synchronize()
    _, _, rp = oracle.route(ids, d["E"])
    rows = np.arange(rp.size) if sample is None else np.sort(
        np.random.default_rng(4).choice(rp.size, min(sample, rp.size), replace=False))
    h_gpu = h.cpu().numpy()[rows]
    q_ref, s_ref, _ = oracle.quantize_rows(h_gpu)
    q_gpu, s_gpu = hq.cpu().numpy()[rows], hs.cpu().numpy()[rows]
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ from the oracle's quantiser on the GPU's h, first {bad[:4].tolist()}"
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32))
    gu64, err = sorted_rows_gate_up(d["qx"], d["sx"], ids, rp, rows, d["q13"], d["s13"], d["k"])
    h32, dh = swiglu_bound(gu64, err)
    over = np.abs(h_gpu.astype(np.float64) - h32) > dh
    assert not over.any(), f"{over.sum()} h values outside the propagated bound"
    rep = {"rows": int(rows.size), "codes": int(q_ref.size), "max_h_err_over_bound":
           float(np.max(np.abs(h_gpu - h32) / dh))}
    print("requant bit-exact", rep, flush=True)
    record(f"moe requant bit-exact on GPU h T={d['T']} E={d['E']} k={d['k']}", rep)


@pytest.mark.parametrize("cfg", ["small", "ragged", "mid"])
def test_requant_bitexact_small(cfg, request):
    _check_requant_bitexact(request.getfixturevalue(cfg))


def test_requant_bitexact_gate_up_cfg(gate_up_cfg):
    """4096 tokens, top-8 of 64 experts: every routed slot's codes and scale."""
    _check_requant_bitexact(gate_up_cfg)


def test_requant_bitexact_large_groups():
    """A 256 x 256-tile shape (2048 rows per group)."""
    d = quantized_moe(**LARGE_GROUPS[3], seed=19)
    _check_requant_bitexact(d, sample=4096)


def test_down_combine_deterministic(small):
    dv = _dev(small)
    ids, tw = small["routes"][0]
    _, offsets, perm = w8.moe_route(to_dev(ids), small["E"], order=0)
    hq, hs = w8.moe_gate_up_swiglu_quant(dv["qx"], dv["sx"], perm, offsets, dv["q13"], dv["s13"], small["k"],
                                         order=0)
    outs = [bf16_bits(w8.moe_down_combine(hq, hs, perm, offsets, to_dev(ids), to_dev(tw), dv["q2"], dv["s2"]))
            for _ in range(3)]
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_down_combine_order_independent(small):
    """The per-slot products and the fixed j order of the combine make the
    output the same, bit for bit, whichever sorted order the rows are in."""
    outs = []
    ids, tw = small["routes"][0]
    dv = _dev(small)
    for order in (0, 1):
        hq, hs, perm, offsets = _check_fused_requant(small, tile_order=order, row_order=order)
        outs.append(bf16_bits(w8.moe_down_combine(hq, hs, perm, offsets, to_dev(ids), to_dev(tw), dv["q2"],
                                                  dv["s2"], order=order)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


def test_down_combine_two_pass_cfg(two_pass_cfg):
    hq, hs, perm, offsets = _check_fused_requant(two_pass_cfg, sample=4096)
    _check_down(two_pass_cfg, hq, hs, perm, offsets, n_tokens=512)


def _oracle_pass_tokens(qx, sx, ids, w, d, tokens):
    out64, _, _ = oracle.moe_pass(qx[tokens], sx[tokens], ids[tokens], w[tokens], d["q13"], d["s13"],
                                  d["q2"], d["s2"])
    return out64


def _check_pass_stagewise(d, dv, qx_ref, sx_ref, xq, xs, ids, tw, full_out, tokens):
    """One routed-expert pass checked stage by stage on ``tokens``, each stage
    fed the GPU's own input of that stage: the full pass's BF16 output must
    equal the stage-by-stage chain (route, gate/up + SwiGLU + requant, down +
    combine) bit for bit; h inside its propagated bound; the requantised codes
    bit-exact on the GPU's h; the down projection + combine inside the element
    bound. ``dv`` holds the device copies of the weights (``_dev``). Returns
    (chain output, its bits, down+combine report, requant report)."""
    ids_d, tw_d = to_dev(ids), to_dev(tw)
    _, off, perm = w8.moe_route(ids_d, d["E"])
    hq, hs, h = w8.moe_gate_up_swiglu_quant(xq, xs, perm, off, dv["q13"], dv["s13"], d["k"], return_h=True)
    out = w8.moe_down_combine(hq, hs, perm, off, ids_d, tw_d, dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    out_bits = bf16_bits(out)
    assert np.array_equal(out_bits, bf16_bits(full_out)), "the full pass differs from the stage-by-stage chain"
    _, _, rp = oracle.route(ids, d["E"])
    inv = np.full(ids.size, -1, np.int64)
    inv[rp] = np.arange(rp.size)
    rows = np.sort(inv[(tokens[:, None] * d["k"] + np.arange(d["k"])[None, :]).reshape(-1)])
    rows = rows[rows >= 0]
    h_gpu = h.cpu().numpy()[rows]
    q_ref, s_ref, _ = oracle.quantize_rows(h_gpu)
    assert np.array_equal(hq.cpu().numpy()[rows], q_ref)
    assert np.array_equal(hs.cpu().numpy()[rows].view(np.uint32), s_ref.view(np.uint32))
    gu64, err = sorted_rows_gate_up(qx_ref, sx_ref, ids, rp, rows, d["q13"], d["s13"], d["k"])
    h32, dh = swiglu_bound(gu64, err)
    assert not (np.abs(h_gpu.astype(np.float64) - h32) > dh).any(), "h outside its bound"
    rq = check_requant(hq.cpu().numpy()[rows], hs.cpu().numpy()[rows], gu64, err)
    ref64, derr = down_combine_ref(hq.cpu().numpy(), hs.cpu().numpy(), perm.cpu().numpy(), ids, tw,
                                   d["q2"], d["s2"], d["k"], tokens)
    rep_dc = bf16_compare(out_bits[tokens], ref64, derr)
    assert rep_dc["n_bound_violations"] == 0, rep_dc
    return out, out_bits, rep_dc, rq


@pytest.mark.parametrize("cfg", ["small", "ragged", "mid"])
def test_full_pass_small(cfg, request):
    d = request.getfixturevalue(cfg)
    dv = _dev(d)
    ids, w = d["routes"][0]
    out = w8.moe_w8a8_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    tokens = np.arange(d["T"])
    _, _, rep_dc, rq = _check_pass_stagewise(d, dv, d["qx"], d["sx"], dv["qx"], dv["sx"], ids, w, out, tokens)
    ref64 = _oracle_pass_tokens(d["qx"], d["sx"], ids, w, d, tokens)
    rep = bf16_compare(bf16_bits(out), ref64)
    rep.update({"down_combine_frobenius": rep_dc["frobenius"], "down_combine_max_abs_over_rms":
                rep_dc["max_abs_over_rms"], "requant_codes_differ_from_oracle": rq["n_codes_differ"],
                "requant_codes": rq["n"]})
    print(f"full pass {cfg}", rep, flush=True)
    record(f"moe full pass {cfg} T={d['T']} H={d['H']} I={d['I']} E={d['E']} k={d['k']}", rep)
    assert rep["frobenius"] <= 4e-3, rep


def test_two_pass_stack(two_pass_cfg):
    """16384 tokens, two passes with the same weights, 512 sampled tokens per pass.

    The benched path (moe_ffn: two moe_w8a8_grouped calls, the next pass's
    input quantised in the first pass's combine) must equal the stage-by-stage
    chain bit for bit; each stage of the chain is then checked element by
    element, each fed the GPU's own input of that stage (teacher forcing):
    the token codes bit-exact, h inside its propagated bound, the requantised
    codes bit-exact on the GPU's h, the down projection + combine inside the
    element bound. End to end, each pass is compared with the oracle's pass
    from the GPU's own input (pass 2 starts from the GPU's pass-1 output)."""
    d = two_pass_cfg
    dv = _dev(d)
    from gpu_util import to_dev_bf16
    x = to_dev_bf16(d["x_bits"])
    routes_dev = [(to_dev(i), to_dev(w)) for i, w in d["routes"]]
    ws = w8.moe_workspace(d["T"], d["H"], d["I"], d["E"], d["k"])
    outs = w8.moe_ffn(x, routes_dev, dv["q13"], dv["s13"], dv["q2"], dv["s2"], workspace=ws)
    torch.cuda.synchronize()
    tokens = np.sort(np.random.default_rng(3).choice(d["T"], 512, replace=False))
    xq, xs = w8.quantize_per_token(x)
    x_bits = d["x_bits"]
    for p, ((ids, tw), (ids_d, tw_d)) in enumerate(zip(d["routes"], routes_dev)):
        print(f"[two-pass] pass {p + 1}", flush=True)
        # the token codes of this pass's input
        qx_ref, sx_ref, _ = oracle.quantize_rows(oracle.bf16_bits_to_f64(x_bits).astype(np.float32))
        assert np.array_equal(xq.cpu().numpy(), qx_ref) and np.array_equal(xs.cpu().numpy(), sx_ref)
        out, out_bits, rep_dc, rq = _check_pass_stagewise(d, dv, qx_ref, sx_ref, xq, xs, ids, tw, outs[p], tokens)
        # end to end against the oracle's pass from the same input
        ref_e2e = _oracle_pass_tokens(qx_ref, sx_ref, ids, tw, d, tokens)
        rep = bf16_compare(out_bits[tokens], ref_e2e)
        rep.update({"down_combine_frobenius": rep_dc["frobenius"], "down_combine_max_abs_over_rms":
                    rep_dc["max_abs_over_rms"], "requant_codes_differ_from_oracle": rq["n_codes_differ"],
                    "requant_codes": rq["n"]})
        print(f"pass {p + 1}", rep, flush=True)
        record(f"moe two-pass T=16384 pass {p + 1} (512 tokens)", rep)
        assert rep["frobenius"] <= 4e-3, rep
        # the next pass's input: the combine's fused quantisation of this output
        if p + 1 < len(d["routes"]):
            _, xq_f, xs_f = w8.moe_w8a8_grouped(xq, xs, ids_d, tw_d, dv["q13"], dv["s13"], dv["q2"], dv["s2"],
                                                quantize_output=True)
            xq, xs = w8.quantize_per_token(out)
            torch.cuda.synchronize()
            assert np.array_equal(xq_f.cpu().numpy(), xq.cpu().numpy())
            assert np.array_equal(xs_f.cpu().numpy(), xs.cpu().numpy())
            x_bits = out_bits


def test_all_slots_dropped_gives_zeros(small):
    dv = _dev(small)
    T, k = small["T"], small["k"]
    ids = np.full((T, k), -1, np.int32)
    w = np.ones((T, k), np.float32)
    out = w8.moe_w8a8_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    assert not bf16_bits(out).any()


def test_partly_dropped_slots(ragged):
    """Some slots dropped (id -1, or an id outside [0, E)), the rest routed:
    the full pass skips exactly those copies. Checked against the oracle's
    pass on every token and against the stage chain bit for bit; every
    token with no valid slot left comes out zero."""
    d = dict(ragged)
    ids, w = d["routes"][0]
    ids = ids.copy()
    ids[::3, 0] = -1
    ids[1::5, -1] = d["E"] + 2
    ids[7] = -1                                   # one token with no valid slot
    d["routes"] = [(ids, w)] + list(d["routes"][1:])
    dv = _dev(d)
    out = w8.moe_w8a8_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    tokens = np.arange(d["T"])
    _check_pass_stagewise(d, dv, d["qx"], d["sx"], dv["qx"], dv["sx"], ids, w, out, tokens)
    rep = bf16_compare(bf16_bits(out), _oracle_pass_tokens(d["qx"], d["sx"], ids, w, d, tokens))
    assert rep["frobenius"] <= 4e-3, rep
    assert not bf16_bits(out)[7].any()


def test_moe_argument_errors(small):
    dv = _dev(small)
    ids = torch.zeros((small["T"], small["k"]), dtype=torch.int32, device="cuda")
    w = torch.ones((small["T"], small["k"]), dtype=torch.float32, device="cuda")
    q13 = torch.zeros((small["E"], 2 * 48, small["H"]), dtype=torch.uint8, device="cuda")
    s13 = torch.ones((small["E"], 2 * 48), dtype=torch.float32, device="cuda")
    q2 = torch.zeros((small["E"], small["H"], 48), dtype=torch.uint8, device="cuda")
    s2 = torch.ones((small["E"], small["H"]), dtype=torch.float32, device="cuda")
    with pytest.raises(w8.W8A8Error) as e:
        w8.moe_w8a8_grouped(dv["qx"], dv["sx"], ids, w, q13, s13, q2, s2)   # I = 48 has no fused kernel
    assert e.value.status == 4


def test_mismatched_order_is_rejected(small):
    """Offsets made in one sorted order cannot be handed to a stage expecting
    the other: the binding checks their length before anything is launched."""
    dv = _dev(small)
    ids, tw = small["routes"][0]
    _, off0, perm0 = w8.moe_route(to_dev(ids), small["E"], order=0)
    with pytest.raises(ValueError):
        w8.moe_gate_up_swiglu_quant(dv["qx"], dv["sx"], perm0, off0, dv["q13"], dv["s13"], small["k"], order=1)
    hq = torch.zeros((small["T"] * small["k"], small["I"]), dtype=torch.uint8, device="cuda")
    hs = torch.ones(small["T"] * small["k"], dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        w8.moe_down_combine(hq, hs, perm0, off0, to_dev(ids), to_dev(tw), dv["q2"], dv["s2"], order=1)


@pytest.mark.parametrize("cfg", [dict(T=37, H=256, I=256, E=5, k=3), dict(T=301, H=272, I=384, E=9, k=4),
                                 dict(T=64, H=2064, I=128, E=4, k=2), dict(T=16, H=8208, I=128, E=3, k=2)])
def test_fused_output_quantisation(cfg):
    """The pass's per-token FP8 output (made in the combine for H <= 8192, by
    a separate quantisation beyond) equals quantize_per_token of its BF16
    output bit for bit, and the oracle's quantiser on the same values."""
    print(f"[fused out quant] {cfg}", flush=True)
    d = quantized_moe(**cfg, n_outlier=2, seed=17)
    dv = _dev(d)
    ids, w = d["routes"][0]
    args = (dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    plain = w8.moe_w8a8_grouped(*args)
    out, q, s = w8.moe_w8a8_grouped(*args, quantize_output=True)
    q2, s2 = w8.quantize_per_token(out)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), bf16_bits(plain))
    assert np.array_equal(q.cpu().numpy(), q2.cpu().numpy())
    assert np.array_equal(s.cpu().numpy(), s2.cpu().numpy())
    qo, so, _ = oracle.quantize_rows(oracle.bf16_bits_to_f64(bf16_bits(out)).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy(), so)


@pytest.mark.parametrize("E", [128, 192])
def test_pages_expert_shapes(E):
    """The model pages' expert shapes (128 or 192 experts, latent width 1024,
    top-4; the intermediate width 512 is a reading): a full pass on 512
    tokens, checked stage by stage and end to end against the oracle on
    every token."""
    print(f"[pages shape] E={E}", flush=True)
    d = quantized_moe(T=512, H=1024, I=512, E=E, k=4, n_outlier=5, seed=E)
    dv = _dev(d)
    ids, w = d["routes"][0]
    out = w8.moe_w8a8_grouped(dv["qx"], dv["sx"], to_dev(ids), to_dev(w), dv["q13"], dv["s13"], dv["q2"], dv["s2"])
    torch.cuda.synchronize()
    tokens = np.arange(d["T"])
    _, _, rep_dc, rq = _check_pass_stagewise(d, dv, d["qx"], d["sx"], dv["qx"], dv["sx"], ids, w, out, tokens)
    ref64 = _oracle_pass_tokens(d["qx"], d["sx"], ids, w, d, tokens)
    rep = bf16_compare(bf16_bits(out), ref64)
    rep.update({"down_combine_frobenius": rep_dc["frobenius"], "requant_codes_differ_from_oracle":
                rq["n_codes_differ"], "requant_codes": rq["n"]})
    print(f"pages shape E={E}", rep, flush=True)
    record(f"moe full pass pages shape T=512 H=1024 I=512 E={E} k=4", rep)
    assert rep["frobenius"] <= 4e-3, rep
