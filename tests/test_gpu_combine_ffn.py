"""GPU parity of moe_combine, moe_combine_bwd and moe_expert_ffn against the CPU
oracle, through the C ABI.  Floating-point outputs: max relative error
(max|got - ref| / max|ref|) <= 2e-2 for bf16 tensors and <= 1e-5 for fp32
tensors; layouts come from the GPU dispatch, which the dispatch tests prove
bit-exact against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_BF16, TOL_F32, dev, host, layout_host, max_rel_err, tol_for, workload_inputs, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def dispatch_case(moe, w: mi.Workload, seed=0):
    idx, wts, logits, x = workload_inputs(w, seed)
    if idx is None:
        idx, wts, _, _ = oracle.route(logits, w.top_k)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), w.n_experts, capacity=w.capacity, max_rows=w.rows)
    return idx, wts, x, xp, lay


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("wid", [1, 2, 3])
def test_combine_identity_expert_full_size(moe, wid):
    w = mi.workload(wid)
    idx, wts, x, xp, lay = dispatch_case(moe, w)
    out = moe.moe_combine(xp, dev(wts), lay)
    got = host(out)
    ref_lay = layout_host(lay)
    ref_lay["rows"] = lay.rows
    ref = oracle.combine(host(xp), wts, ref_lay, w.n_tokens, w.top_k)
    # the kernel takes the oracle's fp32 fused multiply-adds in slot order: equal bits
    np.testing.assert_array_equal(got, ref)
    if wid == 2:
        # identity expert, renormalised weights, nothing dropped: combine(dispatch(x)) == x bit for bit
        assert (got == x).all()
    if wid == 1:
        assert np.abs(values(got) - values(x)).max() <= 4 * 2.0 ** -23 * np.abs(x).max()


@pytest.mark.parametrize("dt", [mi.DT_F32, mi.DT_BF16])
@pytest.mark.parametrize("capacity", [0, 5])
def test_combine_random_rows_with_drops_and_sentinels(moe, dt, capacity):
    g = np.random.default_rng(40 + dt * 2 + (capacity > 0))
    n, e, k, h = 777, 64, 6, 320 if dt == mi.DT_F32 else 640
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.3] = -1
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), dt, 41, 1)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e, capacity=capacity)
    y = mi.normal_activations((lay.rows, h), dt, 41, 2)
    out = moe.moe_combine(dev(y), dev(wts), lay)
    ref_lay = oracle.layout(idx, e, capacity)
    ref = oracle.combine(y, wts, ref_lay, n, k)
    got = host(out)
    np.testing.assert_array_equal(got, ref)   # same fp32 fused multiply-adds in slot order
    none = (ref_lay["assign_row"].reshape(n, k) < 0).all(1)
    assert (got[none].view(np.uint8) == 0).all()


# --------------------------------------------------------- combine backward

def check_combine_bwd(moe, idx, wts, e, capacity, go, y, max_rows=0):
    n, k = idx.shape
    ref_lay = oracle.layout(idx, e, capacity, max_rows)
    x_dummy = np.zeros((n, y.shape[1]), y.dtype)
    _, _, lay = moe.moe_dispatch(dev(x_dummy), dev(idx), dev(wts), e, capacity=capacity, max_rows=max_rows)
    gy, gw = moe.moe_combine_bwd(dev(go), dev(y), dev(wts), lay)
    gy_h, gw_h = host(gy), host(gw)
    ref_gy, ref_gw = oracle.combine_bwd(go, y, wts, ref_lay, k, grad_y=gy_h.copy())
    written = ref_lay["row_src"] >= 0
    if capacity:
        written[:] = True
    assert max_rel_err(gy_h[written], ref_gy[written]) <= tol_for(y)
    assert max_rel_err(gw_h, ref_gw) <= TOL_F32
    assert (gw_h.reshape(-1)[ref_lay["assign_row"] < 0] == 0).all()


@pytest.mark.parametrize("dt", [mi.DT_F32, mi.DT_BF16])
@pytest.mark.parametrize("capacity", [0, 5])
def test_dispatch_bwd_random_rows_with_drops_and_sentinels(moe, dt, capacity):
    g = np.random.default_rng(60 + capacity + dt)
    n, k, e, h = 301, 4, 9, 200
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.2] = -1
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), dt, 61, 1)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e, capacity=capacity)
    lay_h = oracle.layout(idx, e, capacity)
    gxp = mi.normal_activations((lay_h["rows"], h), dt, 62, 2)
    got = host(moe.moe_dispatch_bwd(dev(gxp), lay))
    ref = oracle.dispatch_bwd(gxp, lay_h, n, k)
    # same fp32 adds in the same slot order, one rounding: bit for bit
    assert (got.view(np.uint8) == ref.view(np.uint8)).all()


@pytest.mark.parametrize("wid", [2, 3])
def test_dispatch_bwd_full_size(moe, wid):
    w = mi.workload(wid)
    idx, wts, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    lay_h = oracle.layout(idx, w.n_experts, w.capacity)
    x = mi.activations(w)
    _, _, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), w.n_experts, capacity=w.capacity)
    gxp = mi.normal_activations((lay_h["rows"], w.hidden), mi.DT_BF16, 63, 3)
    got = host(moe.moe_dispatch_bwd(dev(gxp), lay))
    ref = oracle.dispatch_bwd(gxp, lay_h, w.n_tokens, w.top_k)
    assert (got.view(np.uint8) == ref.view(np.uint8)).all()


def test_dispatch_bwd_empty(moe):
    idx = np.zeros((0, 2), np.int32)
    x = np.zeros((0, 64), np.float32)
    _, _, lay = moe.moe_dispatch(dev(x), dev(idx), dev(np.zeros((0, 2), np.float32)), 4)
    out = moe.moe_dispatch_bwd(dev(np.zeros((0, 64), np.float32)), lay)
    assert tuple(out.shape) == (0, 64)


@pytest.mark.parametrize("dt", [mi.DT_F32, mi.DT_BF16])
@pytest.mark.parametrize("capacity", [0, 7])
def test_combine_bwd_small(moe, dt, capacity):
    g = np.random.default_rng(60 + dt + capacity)
    n, e, k, h = 501, 32, 4, 384
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.2] = -1
    wts = g.random((n, k)).astype(np.float32)
    rows = e * capacity if capacity else n * k
    go = mi.normal_activations((n, h), dt, 61, 1)
    y = mi.normal_activations((rows, h), dt, 61, 2)
    check_combine_bwd(moe, idx, wts, e, capacity, go, y)


def test_combine_bwd_expert_share_full_size(moe):
    w = mi.workload(5)
    idx, wts = mi.received_routing(w)
    go = mi.grad_output(w)
    y = mi.normal_activations((w.rows, w.hidden), mi.DT_BF16, 5, 9)
    check_combine_bwd(moe, idx, wts, w.n_experts, 0, go, y, max_rows=w.rows)


# --------------------------------------------------------------- expert FFN

def ffn_case(moe, n, e, k, h, inter, capacity=0, seed=0, zero_expert=None):
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter,
                    capacity_factor=0.0 if not capacity else capacity)
    logits = mi.router_logits(w, seed)
    if zero_expert is not None:
        logits[:, zero_expert] = -50.0
    idx, wts, _, _ = oracle.route(logits, k)
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e, capacity=w.capacity)
    y = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd))
    torch.cuda.synchronize()
    return w, idx, wts, x, wgu, wd, xp, lay, y


@pytest.mark.parametrize("n,e,k,h,inter,cap", [
    (300, 4, 2, 256, 192, 0),     # several m-tiles per expert, ragged tails
    (257, 8, 2, 192, 128, 0),     # hidden not a multiple of 128 (masked columns)
    (1000, 16, 4, 512, 256, 0),
    (600, 8, 2, 256, 64, 1.0),    # capacity layout with drops and pads
    (5, 4, 1, 64, 64, 0),         # tiny, most experts empty
])
def test_expert_ffn_small_full_compare(moe, n, e, k, h, inter, cap):
    w, idx, wts, x, wgu, wd, xp, lay, y = ffn_case(moe, n, e, k, h, inter, cap, zero_expert=1 if e > 2 else None)
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    ref = oracle.expert_ffn(host(xp), lay_h, wgu, wd)
    got = host(y)
    kept = lay_h["pad_mask"] == 0
    assert kept.sum() == lay_h["counters"][0]
    assert max_rel_err(got[kept], ref[kept]) <= TOL_BF16
    # most outputs should round to the same bf16 value
    assert (got[kept] == ref[kept]).mean() > 0.9


# ------------------------------------------------------ expert FFN backward

def ffn_bwd_run(moe, w, xp, lay, wgu, wd, seed=0):
    dy = mi.grad_expert_rows(w, lay.rows, seed)
    gx, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, dev(dy), lay, dev(wgu), dev(wd))
    torch.cuda.synchronize()
    return dy, gx, dwgu, dwd


def entries(t: torch.Tensor, idx) -> np.ndarray:
    """Elements idx (a list of index tuples) of a device tensor, gathered on the device."""
    cols = [torch.tensor(c, dtype=torch.long, device=t.device) for c in zip(*idx)]
    return host(t[tuple(cols)].contiguous())


@pytest.mark.parametrize("n,e,k,h,inter,cap", [
    (300, 4, 2, 256, 192, 0),     # several m-tiles per expert, ragged tails
    (257, 8, 2, 192, 128, 0),     # hidden not a multiple of 128 (masked columns and weight-gradient rows)
    (1000, 16, 4, 512, 256, 0),
    (2000, 4, 2, 128, 320, 0),    # long expert segments: many K steps in the weight gradients
    (600, 8, 2, 256, 64, 1.0),    # capacity layout with drops and pads
    (5, 4, 1, 64, 64, 0),         # tiny, most experts empty
    (300, 1, 1, 256, 192, 0),     # one expert: its weight-gradient tiles split over the XCDs
    (400, 2, 1, 512, 256, 0),     # two experts
    (2048, 64, 2, 1024, 512, 0),  # whole tiles of one or two K steps, several per workgroup in a row
])
def test_expert_ffn_bwd_small_full_compare(moe, n, e, k, h, inter, cap):
    w, idx, wts, x, wgu, wd, xp, lay, y = ffn_case(moe, n, e, k, h, inter, cap, zero_expert=1 if e > 2 else None)
    dy, gx, dwgu, dwd = (host(v) if isinstance(v, torch.Tensor) else v for v in ffn_bwd_run(moe, w, xp, lay, wgu, wd))
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    ref_gx, ref_dwgu, ref_dwd = oracle.expert_ffn_bwd(host(xp), dy, lay_h, wgu, wd)
    cnt, offs = lay_h["tokens_per_expert"], lay_h["expert_offsets"]
    in_seg = np.zeros(lay.rows, bool)
    for ex in range(e):
        in_seg[offs[ex]:offs[ex] + cnt[ex]] = True
    assert max_rel_err(gx[in_seg], ref_gx[in_seg]) <= TOL_BF16
    assert max_rel_err(dwgu, ref_dwgu) <= TOL_BF16
    assert max_rel_err(dwd, ref_dwd) <= TOL_BF16
    for ex in np.nonzero(cnt == 0)[0]:          # experts without rows: exactly zero weight gradients
        assert (dwgu[ex] == 0).all() and (dwd[ex] == 0).all()
    if e > 2:
        assert cnt[1] == 0


def test_expert_ffn_and_bwd_empty(moe):
    """No rows: the forward writes nothing, the backward gives zero weight gradients."""
    e, h, inter = 4, 128, 64
    x = torch.empty((0, h), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    wts = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    xp, wp, lay = moe.moe_dispatch(x, idx, wts, e)
    g = torch.Generator(device="cuda").manual_seed(0)
    wgu = torch.randn((e, 2 * inter, h), generator=g, device="cuda").to(torch.bfloat16)
    wd = torch.randn((e, h, inter), generator=g, device="cuda").to(torch.bfloat16)
    y = moe.moe_expert_ffn(xp, lay, wgu, wd)
    gx, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, torch.empty_like(xp), lay, wgu, wd,
                                           grad_w_gate_up=torch.full_like(wgu, 3.0), grad_w_down=torch.full_like(wd, 3.0))
    torch.cuda.synchronize()
    assert y.shape == (0, h) and gx.shape == (0, h)
    assert not dwgu.view(torch.int16).any() and not dwd.view(torch.int16).any()


def test_expert_ffn_and_bwd_1024_experts(moe):
    """The most experts the tile scan takes, most of them empty, a few with ragged rows."""
    n, e, k, h, inter = 600, 1024, 2, 128, 64
    w, idx, wts, x, wgu, wd, xp, lay, y = ffn_case(moe, n, e, k, h, inter)
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    ref = oracle.expert_ffn(host(xp), lay_h, wgu, wd)
    kept = lay_h["pad_mask"] == 0
    assert max_rel_err(host(y)[kept], ref[kept]) <= TOL_BF16
    dy, gx, dwgu, dwd = (host(v) if isinstance(v, torch.Tensor) else v for v in ffn_bwd_run(moe, w, xp, lay, wgu, wd))
    ref_gx, ref_dwgu, ref_dwd = oracle.expert_ffn_bwd(host(xp), dy, lay_h, wgu, wd)
    assert max_rel_err(gx[kept], ref_gx[kept]) <= TOL_BF16
    assert max_rel_err(dwgu, ref_dwgu) <= TOL_BF16 and max_rel_err(dwd, ref_dwd) <= TOL_BF16


def test_expert_ffn_bwd_repeated_calls_are_identical(moe):
    """The backward is deterministic: no atomics, fixed reduction order."""
    w, idx, wts, x, wgu, wd, xp, lay, y = ffn_case(moe, 700, 8, 2, 256, 128)
    a = ffn_bwd_run(moe, w, xp, lay, wgu, wd)
    b = ffn_bwd_run(moe, w, xp, lay, wgu, wd)
    for u, v in zip(a[1:], b[1:]):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("n,e,k,h,inter,cap", [
    (300, 4, 2, 256, 192, 0),
    (600, 8, 2, 256, 64, 1.0),
])
def test_expert_ffn_saved_gate_up(moe, n, e, k, h, inter, cap):
    """The forward's stored pre-activations match the oracle, leave y unchanged,
    and the backward that takes them gives the same bits as the one recomputing them."""
    w, idx, wts, x, wgu, wd, xp, lay, y = ffn_case(moe, n, e, k, h, inter, cap, zero_expert=1)
    y2, gu = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd), save_gate_up=True)
    torch.cuda.synchronize()
    lay_h = layout_host(lay)
    rows = np.nonzero(lay_h["pad_mask"] == 0)[0]
    sel = torch.as_tensor(rows, device=y.device)
    assert torch.equal(y[sel].view(torch.int16), y2[sel].view(torch.int16))   # rows outside the segments: unwritten
    ref = oracle.expert_gate_up_rows(rows, host(xp), lay_h, wgu)
    got = host(gu)[rows]
    assert max_rel_err(got, ref) <= TOL_BF16
    assert (got == ref).mean() > 0.9
    dy = dev(mi.grad_expert_rows(w, lay.rows))
    saved = gu.clone()
    a = moe.moe_expert_ffn_bwd(xp, dy, lay, dev(wgu), dev(wd))
    b = moe.moe_expert_ffn_bwd(xp, dy, lay, dev(wgu), dev(wd), gate_up=gu)
    torch.cuda.synchronize()
    assert torch.equal(a[0][sel].view(torch.int16), b[0][sel].view(torch.int16))   # grad_x_perm, segment rows
    for u, v in zip(a[1:], b[1:]):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
    assert torch.equal(saved.view(torch.int16), gu.view(torch.int16))   # the saved buffer is only read


def test_layer_step_replays_in_a_hip_graph(moe):
    """route -> dispatch -> grouped FFN -> combine captured once in a HIP graph (the
    library launches kernels only: no memsets, allocations or host synchronisation)
    and replayed three times, with other work and synchronisation in between; every
    replay equals the eager step bit for bit."""
    n, e, k, h, inter = 512, 16, 4, 256, 128
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter)
    logits, x = dev(mi.router_logits(w)), dev(mi.activations(w))
    wgu, wd = (dev(a) for a in mi.expert_weights(w))
    r = moe.moe_route(logits, k)
    xp, wp, lay = moe.moe_dispatch(x, r.topk_idx, r.topk_w, e)
    y = torch.empty_like(xp)
    out = torch.empty_like(x)
    shape_d = moe.make_shape(n, h, e, k)
    ws_d = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape_d, "cuda")
    ws_f = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN, lay.shape(h, moe.MOE_DT_BF16, inter), "cuda")

    def step():
        moe.moe_route(logits, k, out=r)
        moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, layout=lay, x_perm=xp, w_perm_out=wp, workspace=ws_d)
        moe.moe_expert_ffn(xp, lay, wgu, wd, y=y, workspace=ws_f)
        moe.moe_combine(y, r.topk_w, lay, out=out)

    step()
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_idx = r.topk_idx.clone()
    ref_rows = lay.assign_row.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(7.0)
        lay.assign_row.fill_(-5)
        r.topk_idx.fill_(-5)
        torch.randn(1 << 20, device="cuda").sum()       # other work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), i
        assert torch.equal(r.topk_idx, ref_idx) and torch.equal(lay.assign_row, ref_rows), i
