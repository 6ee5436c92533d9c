"""GPU parity of moe_route and moe_dispatch against the CPU oracle, through the
C ABI.  Bit-exact: top-k indices, routing map, counts, every layout array,
dispatched rows and permuted weights.  Router weights: max relative error
<= 1e-5 (fp32)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_BF16, TOL_F32, assert_layout_equal, dev, host, layout_host, max_rel_err, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def check_route(moe, logits: np.ndarray, k: int):
    r = moe.moe_route(dev(logits), k)
    torch.cuda.synchronize()
    idx, w, rmap, tpe = oracle.route(logits, k)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.routing_map), rmap)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    if not np.isnan(logits).any() and idx.size:
        assert max_rel_err(host(r.topk_w), w) <= TOL_F32
    return r


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_route_workloads_full_size(moe, wid):
    w = mi.workload(wid)
    check_route(moe, mi.router_logits(w), w.top_k)


@pytest.mark.parametrize("e,k", [(8, 1), (8, 8), (64, 2), (100, 7), (256, 8), (300, 5), (1024, 16), (1000, 1000)])
def test_route_shapes_ties_signed_zero_nan(moe, e, k):
    g = np.random.default_rng(e * 31 + k)
    n = 1003 if e * k < 100000 else 37
    logits = g.standard_normal((n, e)).astype(np.float32)
    check_route(moe, logits, k)
    vals = np.array([-1.0, -0.0, 0.0, 1.0, np.nan], np.float32)
    ties = g.choice(vals, size=(n, e), p=[0.25, 0.2, 0.2, 0.25, 0.1]).astype(np.float32)
    check_route(moe, ties, k)


@pytest.mark.parametrize("e,k,with_map", [(8, 2, True), (100, 7, True), (256, 8, True), (256, 8, False), (1024, 16, True)])
def test_route_token_mask(moe, e, k, with_map):
    """Padding tokens route nowhere; both counting paths (map column sums, and the
    router's own histogram when there is no map or E % 16 != 0)."""
    g = np.random.default_rng(e + k)
    n = 777
    logits = g.standard_normal((n, e)).astype(np.float32)
    mask = (g.random(n) < 0.25).astype(np.uint8)
    r = moe.moe_route(dev(logits), k, token_mask=dev(mask), routing_map=with_map)
    torch.cuda.synchronize()
    idx, w, rmap, tpe = oracle.route(logits, k, mask)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    if with_map:
        np.testing.assert_array_equal(host(r.routing_map), rmap)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    got_w = host(r.topk_w)
    assert (got_w[mask == 1] == 0).all()
    assert max_rel_err(got_w, w) <= TOL_F32


@pytest.mark.parametrize("e,k,ties", [(8, 2, False), (100, 7, True), (256, 8, False), (256, 8, True), (1000, 70, False)])
def test_route_expert_bias(moe, e, k, ties):
    """Selection by logit + bias, weights from the logits; with ties between biased scores."""
    g = np.random.default_rng(7 * e + k)
    n = 513
    logits = g.standard_normal((n, e)).astype(np.float32)
    bias = (g.standard_normal(e) * 0.5).astype(np.float32)
    if ties:
        logits = (np.round(logits * 2) / 2).astype(np.float32)
        bias = np.round(bias).astype(np.float32)
    mask = (g.random(n) < 0.1).astype(np.uint8)
    r = moe.moe_route(dev(logits), k, expert_bias=dev(bias), token_mask=dev(mask))
    torch.cuda.synchronize()
    idx, w, rmap, tpe = oracle.route(logits, k, mask, bias)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.routing_map), rmap)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    assert max_rel_err(host(r.topk_w), w) <= TOL_F32


def test_route_expert_bias_balances_skewed_logits(moe):
    """The Zipf-skewed workload's logits with the negated per-expert mean offset as
    the bias: the load evens out (selection), the weights keep the skewed logits."""
    w = mi.workload(3)
    logits = mi.router_logits(w)
    col = logits.astype(np.float64).mean(0)
    bias = (-(col - col.mean())).astype(np.float32)       # undoes the calibrated per-expert skew
    r = moe.moe_route(dev(logits), w.top_k, expert_bias=dev(bias))
    torch.cuda.synchronize()
    idx, wts, _, tpe = oracle.route(logits, w.top_k, expert_bias=bias)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    assert max_rel_err(host(r.topk_w), wts) <= TOL_F32
    skewed = oracle.route(logits, w.top_k)[3]
    assert tpe.max() < skewed.max() / 4                  # 4096 for the hottest expert without the bias


@pytest.mark.parametrize("n,e,k,seed", [(4096, 256, 8, 1), (8192, 128, 8, 2 ** 40 + 3), (777, 100, 7, 0),
                                         (64, 8, 2, 2 ** 64 - 1), (300, 1000, 70, 5)])
def test_route_random_force_balanced(moe, n, e, k, seed):
    """The device-drawn logits and everything derived from them equal the oracle's."""
    r = moe.moe_route_random(n, e, k, seed)
    torch.cuda.synchronize()
    idx, w, rmap, tpe = oracle.route_random(n, e, k, seed)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.routing_map), rmap)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    assert max_rel_err(host(r.topk_w), w) <= TOL_F32
    if n * k >= 32 * e:                                  # balanced: no expert far from N*k/E
        m = n * k / e
        assert tpe.max() < m + 6 * np.sqrt(m) and tpe.min() > m - 6 * np.sqrt(m)


def test_route_random_with_bias_and_mask(moe):
    g = np.random.default_rng(3)
    n, e, k = 1000, 64, 4
    bias = (g.standard_normal(e) * 0.1).astype(np.float32)
    mask = (g.random(n) < 0.2).astype(np.uint8)
    r = moe.moe_route_random(n, e, k, 99, expert_bias=dev(bias), token_mask=dev(mask))
    torch.cuda.synchronize()
    idx, w, rmap, tpe = oracle.route_random(n, e, k, 99, mask, bias)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    assert max_rel_err(host(r.topk_w), w) <= TOL_F32


def test_route_token_mask_through_the_layer(moe):
    """masked route -> dispatch -> combine: padding tokens are not dispatched and get zero rows."""
    w = mi.workload(2, n_tokens=512)
    logits = mi.router_logits(w)
    x = mi.activations(w)
    mask = np.zeros(w.n_tokens, np.uint8)
    mask[::3] = 1
    r = moe.moe_route(dev(logits), w.top_k, token_mask=dev(mask))
    xp, wp, lay = moe.moe_dispatch(dev(x), r.topk_idx, r.topk_w, w.n_experts)
    out = moe.moe_combine(xp, r.topk_w, lay)
    torch.cuda.synchronize()
    idx, wts, _, _ = oracle.route(logits, w.top_k, mask)
    ref_lay = oracle.layout(idx, w.n_experts)
    assert_layout_equal(layout_host(lay), ref_lay)
    assert int(host(lay.counters)[0]) == (1 - mask).sum() * w.top_k
    out_h = host(out)
    assert (out_h[mask == 1] == 0).all()
    xp_ref, _ = oracle.scatter(x, w.top_k, ref_lay, wts)
    ref = oracle.combine(xp_ref, wts, ref_lay, w.n_tokens, w.top_k)
    assert max_rel_err(out_h, ref) <= TOL_BF16


def test_route_empty(moe):
    r = moe.moe_route(torch.empty((0, 16), dtype=torch.float32, device="cuda"), 4)
    torch.cuda.synchronize()
    assert (host(r.tokens_per_expert) == 0).all()


def run_dispatch(moe, x: np.ndarray, idx: np.ndarray, wts: np.ndarray, e: int, capacity=0, max_rows=0, row_align=0,
                 drop_policy=0):
    x_d = dev(x)
    xp, wp, lay = moe.moe_dispatch(x_d, dev(idx), dev(wts), e, capacity=capacity, max_rows=max_rows,
                                   row_align=row_align, drop_policy=drop_policy)
    torch.cuda.synchronize()
    return xp, wp, lay


def check_dispatch(moe, x, idx, wts, e, capacity=0, max_rows=0, row_align=0, drop_policy=0):
    xp, wp, lay = run_dispatch(moe, x, idx, wts, e, capacity, max_rows, row_align, drop_policy)
    ref = oracle.layout(idx, e, capacity, max_rows, row_align, drop_policy, wts)
    got = layout_host(lay)
    assert_layout_equal(got, ref)
    xp_h = host(xp)
    k = idx.shape[1]
    kept = np.nonzero(ref["assign_row"] >= 0)[0]
    rows = ref["assign_row"][kept]
    # dispatched rows: bit-exact copies; capacity pads: all-zero bits
    assert (xp_h[rows].view(np.uint8) == x[kept // k].view(np.uint8)).all()
    if capacity > 0 or row_align > 1:   # capacity or alignment pads: all-zero bits
        pads = np.nonzero(ref["row_src"][:ref["expert_offsets"][-1]] < 0)[0]
        assert (xp_h[pads].view(np.uint8) == 0).all()
    ref_xp, ref_wp = oracle.scatter(x, k, ref, wts, x_perm=xp_h.copy())
    np.testing.assert_array_equal(host(wp), ref_wp)
    assert (xp_h.view(np.uint8) == ref_xp.view(np.uint8)).all()
    return xp, wp, lay, ref


@pytest.mark.parametrize("case", ["random", "ties", "nan", "one_hot_expert", "under_capacity"])
def test_dispatch_drop_by_weight(moe, case):
    """Capacity with the drop-by-weight policy: the radix select keeps each
    expert's largest weights, ties to the earlier assignment."""
    g = np.random.default_rng(["random", "ties", "nan", "one_hot_expert", "under_capacity"].index(case))
    n, e, k, h, cap = 2000, 64, 4, 256, 96
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    wts = g.random((n, k)).astype(np.float32)
    if case == "ties":
        wts = (np.round(wts * 8) / 8).astype(np.float32)
    if case == "nan":
        wts[g.random(wts.shape) < 0.05] = np.nan
        wts[g.random(wts.shape) < 0.05] = -0.0
    if case == "one_hot_expert":
        idx[:, 0] = 5                                   # expert 5 receives every token: 2000 rows for 96 slots
    if case == "under_capacity":
        cap = 400                                       # nobody over capacity: same as the position policy
    x = mi.normal_activations((n, h), mi.DT_BF16, 78, 1)
    xp, wp, lay, ref = check_dispatch(moe, x, idx, wts, e, cap, drop_policy=1)
    if case == "under_capacity":
        assert_layout_equal(layout_host(lay), oracle.layout(idx, e, cap))


def test_dispatch_drop_by_weight_zipf_workload(moe):
    w = mi.workload(3)
    logits = mi.router_logits(w)
    idx, wts, _, _ = oracle.route(logits, w.top_k)
    x = mi.activations(w)
    xp, wp, lay, ref = check_dispatch(moe, x, idx, wts, w.n_experts, w.capacity, drop_policy=1)
    # the kept mass: dropping by weight keeps at least as much routing weight as dropping by position
    kept_w = np.nansum(np.where(ref["assign_row"].reshape(idx.shape) >= 0, wts, 0))
    pos = oracle.layout(idx, w.n_experts, w.capacity)
    kept_pos = np.nansum(np.where(pos["assign_row"].reshape(idx.shape) >= 0, wts, 0))
    assert kept_w > kept_pos


@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_dispatch_workloads_full_size(moe, wid):
    w = mi.workload(wid)
    idx, wts, logits, x = workload_inputs(w)
    if idx is None:
        idx, wts, _, _ = oracle.route(logits, w.top_k)
    check_dispatch(moe, x, idx, wts, w.n_experts, w.capacity, w.rows)


EDGE_CASES = ["ragged", "capacity", "clip_rows", "invalid_ids", "one_expert", "all_to_one", "capacity_one", "k1",
              "e1024", "sentinels", "align64", "align16_clip_rows", "align256_e1024", "align8_capacity"]


@pytest.mark.parametrize("case", EDGE_CASES)
def test_dispatch_edge_cases(moe, case):
    g = np.random.default_rng(100 + EDGE_CASES.index(case))
    n, e, k, h, cap, max_rows, align = 1001, 256, 8, 512, 0, 0, 0
    if case == "one_expert":
        e, k = 1, 1
    if case == "k1":
        k = 1
    if case in ("e1024", "align256_e1024"):
        e = 1024
    if case.startswith("align"):
        align = int(case[5:].split("_")[0])
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if case == "capacity":
        cap = 30
    if case in ("clip_rows", "align16_clip_rows"):
        max_rows = n * k - 777
    if case == "align8_capacity":
        cap = 24
    if case == "invalid_ids":
        bad = g.random(idx.shape) < 0.05
        idx[bad] = g.choice([-5, e, e + 100, -2], size=bad.sum())
    if case == "all_to_one":
        idx[:, 0] = 3
        idx[:, 1:] = -1
    if case == "capacity_one":
        cap = 1
    if case == "sentinels":
        idx[g.random(idx.shape) < 0.75] = -1
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), mi.DT_BF16, 77, 1)
    check_dispatch(moe, x, idx, wts, e, cap, max_rows, align)


@pytest.mark.parametrize("align", [16, 256])
def test_aligned_segments_through_ffn_and_combine_bwd(moe, align):
    """Aligned segments feed the grouped FFN unchanged (its rows are the kept
    rows); combine backward zeroes the alignment pads of grad_y."""
    w = mi.workload(4, n_tokens=512, hidden=256, n_experts=16, inter=128)
    logits = mi.router_logits(w)
    idx, wts, _, _ = oracle.route(logits, w.top_k)
    x = mi.activations(w)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), w.n_experts, row_align=align)
    wgu, wd = mi.expert_weights(w)
    y = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd))
    go = mi.grad_output(w)
    gy, gw = moe.moe_combine_bwd(dev(go), y, dev(wts), lay)
    torch.cuda.synchronize()
    ref_lay = oracle.layout(idx, w.n_experts, row_align=align)
    ref_lay["rows"] = lay.rows
    assert_layout_equal(layout_host(lay), ref_lay)
    kept = ref_lay["pad_mask"] == 0
    ref_y = oracle.expert_ffn(host(xp), ref_lay, wgu, wd)
    y_h = host(y)
    assert max_rel_err(y_h[kept], ref_y[kept]) <= TOL_BF16
    ref_gy, ref_gw = oracle.combine_bwd(go, y_h, wts, ref_lay, w.top_k, grad_y=host(gy).copy())
    used = np.arange(lay.rows) < ref_lay["expert_offsets"][-1]
    gy_h = host(gy)
    assert (gy_h[used & ~kept] == 0).all()                      # alignment pads of grad_y
    assert max_rel_err(gy_h[kept], ref_gy[kept]) <= TOL_BF16
    assert max_rel_err(host(gw), ref_gw) <= TOL_F32


def test_dispatch_fp32_tiny_and_empty(moe):
    g = np.random.default_rng(5)
    idx = np.stack([g.permutation(8)[:2] for _ in range(64)]).astype(np.int32)
    x = mi.normal_activations((64, 128), mi.DT_F32, 1, 1)
    check_dispatch(moe, x, idx, g.random((64, 2)).astype(np.float32), 8)
    check_dispatch(moe, x[:0], idx[:0], np.zeros((0, 2), np.float32), 8)
    check_dispatch(moe, x[:0], idx[:0], np.zeros((0, 2), np.float32), 8, capacity=3)


def test_dispatch_deterministic_and_no_out_of_bounds_writes(moe):
    w = mi.workload(3, n_tokens=2048, hidden=256)
    logits = mi.router_logits(w)
    idx, wts, _, _ = oracle.route(logits, w.top_k)
    x = mi.activations(w)
    rows = w.max_rows
    guard = 4096
    buf = torch.full((rows * w.hidden + 2 * guard,), 7, dtype=torch.int16, device="cuda")
    xp = buf[guard:guard + rows * w.hidden].view(torch.bfloat16).view(rows, w.hidden)
    a = moe.moe_dispatch(dev(x), dev(idx), dev(wts), w.n_experts, capacity=w.capacity, x_perm=xp)
    first = host(xp).copy()
    lay1 = layout_host(a[2])
    b = moe.moe_dispatch(dev(x), dev(idx), dev(wts), w.n_experts, capacity=w.capacity, x_perm=xp)
    torch.cuda.synchronize()
    assert (host(xp) == first).all()
    assert_layout_equal(layout_host(b[2]), lay1)
    hb = host(buf)
    assert (hb[:guard] == 7).all() and (hb[-guard:] == 7).all()


def test_route_then_dispatch_on_device(moe):
    """Route output feeds dispatch without leaving the GPU (uniform workload shape)."""
    w = mi.workload(2)
    logits = mi.router_logits(w)
    x = mi.activations(w)
    r = moe.moe_route(dev(logits), w.top_k)
    xp, wp, lay = moe.moe_dispatch(dev(x), r.topk_idx, r.topk_w, w.n_experts)
    torch.cuda.synchronize()
    idx, wts, _, _ = oracle.route(logits, w.top_k)
    assert_layout_equal(layout_host(lay), oracle.layout(idx, w.n_experts))
