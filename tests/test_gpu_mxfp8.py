"""GPU parity of the MXFP8 calls against the CPU oracle, through the C ABI.
moe_dispatch_mxfp8 and moe_mx_quantize bit-exact (every layout array, every
E4M3 code byte and E8M0 scale byte, the permuted weights, the zeroed pad rows);
moe_expert_ffn_mxfp8 within the bf16 tolerance on sampled rows; graph replay of
the MXFP8 and the replicated layer steps bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import (TOL_BF16, assert_layout_equal, dev, every_value_at_every_scale, host, layout_host,
                         max_rel_err, values, workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def check_mx_dispatch(moe, x, idx, wts, e, capacity=0, max_rows=0, row_align=0, drop_policy=0):
    q, sc, wp, lay = moe.moe_dispatch_mxfp8(dev(x), dev(idx), dev(wts), e, capacity=capacity, max_rows=max_rows,
                                            row_align=row_align, drop_policy=drop_policy)
    torch.cuda.synchronize()
    ref = oracle.layout(idx, e, capacity, max_rows, row_align, drop_policy, wts)
    assert_layout_equal(layout_host(lay), ref)
    q_h, sc_h = host(q), host(sc)
    # rows of an unused dropless tail are not written: the oracle keeps what the GPU left there
    ref_q, ref_sc, ref_wp = oracle.dispatch_mxfp8(x, idx.shape[1], ref, wts, x_perm_q=q_h.copy(),
                                                  x_perm_scale=sc_h.copy())
    np.testing.assert_array_equal(sc_h, ref_sc)
    np.testing.assert_array_equal(q_h, ref_q)
    np.testing.assert_array_equal(host(wp), ref_wp)
    return q_h, sc_h, ref


@pytest.mark.parametrize("n,h,e,k", [(300, 256, 16, 4), (1001, 7168, 256, 8), (513, 4096, 128, 8), (77, 32, 3, 2),
                                     (129, 9216, 8, 1), (64, 11264, 64, 12)])
def test_mx_dispatch_shapes(moe, n, h, e, k):
    """Several tiles of blocks per row, rows longer than one workgroup's 256
    blocks (H = 9216, 11264), k not a multiple of the slot chunk."""
    g = np.random.default_rng(n + h + e + k)
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), mi.DT_BF16, 91, n)
    check_mx_dispatch(moe, x, idx, wts, e)


@pytest.mark.parametrize("order", ["shuffled", "by_magnitude"])
def test_mx_dispatch_every_bf16_value(moe, order):
    """Every finite bf16 bit pattern, in blocks of mixed magnitudes (small
    elements rounded into E4M3's subnormals or to signed zero) and in blocks of
    similar magnitudes (every scale code, the clipped smallest scale included)."""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]                                # 65280 finite patterns
    if order == "shuffled":
        b = np.random.default_rng(3).permutation(b)
    else:
        b = b[np.argsort(b & 0x7FFF, kind="stable")]
    x = b.reshape(-1, 256)                                          # 255 token rows
    n = x.shape[0]
    idx = np.stack([np.arange(n) % 5, (np.arange(n) + 2) % 5], axis=1).astype(np.int32)
    wts = np.ones((n, 2), np.float32)
    q, sc, ref = check_mx_dispatch(moe, x, idx, wts, 5)
    if order == "by_magnitude":
        assert {0, 1, 119, 127} <= set(np.unique(sc).tolist())


@pytest.mark.parametrize("case", ["capacity", "capacity_by_weight", "align64", "align16_clip_rows", "sentinels",
                                  "invalid_ids", "clip_rows", "zero_rows"])
def test_mx_dispatch_edge_cases(moe, case):
    g = np.random.default_rng(200 + len(case))
    n, e, k, h, cap, max_rows, align, policy = 1001, 64, 8, 512, 0, 0, 0, 0
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if case.startswith("capacity"):
        cap = 128                                                   # about 125 per expert: drops and pads
        policy = 1 if case.endswith("by_weight") else 0
    if case.startswith("align"):
        align = int(case[5:].split("_")[0])
    if case.endswith("clip_rows"):
        max_rows = n * k - 555
    if case == "sentinels":
        idx[g.random(idx.shape) < 0.75] = -1
    if case == "invalid_ids":
        bad = g.random(idx.shape) < 0.05
        idx[bad] = g.choice([-5, e, e + 100, -2], size=bad.sum())
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), mi.DT_BF16, 92, 1)
    if case == "zero_rows":
        x[::3] = 0
        x[1::3, :64] = 0x8000                                       # -0.0: code 0x80, scale code 0
    q, sc, ref = check_mx_dispatch(moe, x, idx, wts, e, cap, max_rows, align, policy)
    if cap or align:
        pads = np.nonzero(ref["row_src"][:ref["expert_offsets"][-1]] < 0)[0]
        assert pads.size and not q[pads].any() and not sc[pads].any()
    if cap:
        assert ref["counters"][1] > 0                               # some assignments dropped


def test_mx_dispatch_empty(moe):
    x = np.zeros((0, 256), np.uint16)
    idx = np.zeros((0, 2), np.int32)
    wts = np.zeros((0, 2), np.float32)
    check_mx_dispatch(moe, x, idx, wts, 8)
    q, sc, ref = check_mx_dispatch(moe, x, idx, wts, 8, capacity=3)
    assert not q.any() and not sc.any()


@pytest.mark.parametrize("wid", [2, 3, 5])
def test_mx_dispatch_full_size(moe, wid):
    """Full-size workloads (uniform dropless; Zipf with capacity; the expert
    share with -1 sentinels and a row limit): the layout equals the bf16
    dispatch's, every kept row equals the oracle's quantisation of its token
    row byte for byte, and the dequantised rows lie within half an E4M3 grid
    step of the bf16 rows of moe_dispatch (clamped elements within their clamp
    distance)."""
    w = mi.workload(wid)
    idx, wts, logits, x = workload_inputs(w)
    if idx is None:
        idx, wts, _, _ = oracle.route(logits, w.top_k)
    x_d, idx_d, w_d = dev(x), dev(idx), dev(wts)
    q, sc, wp, lay = moe.moe_dispatch_mxfp8(x_d, idx_d, w_d, w.n_experts, capacity=w.capacity, max_rows=w.rows)
    xp, wp16, lay16 = moe.moe_dispatch(x_d, idx_d, w_d, w.n_experts, capacity=w.capacity, max_rows=w.rows)
    torch.cuda.synchronize()
    got = layout_host(lay)
    assert_layout_equal(got, layout_host(lay16))
    assert torch.equal(wp, wp16)
    k = w.top_k
    ref_q, ref_sc = oracle.mx_quantize(x)
    rows = np.nonzero(got["row_src"] >= 0)[0]
    tok = got["row_src"][rows] // k
    q_h, sc_h = host(q), host(sc)
    bad = np.nonzero((q_h[rows] != ref_q[tok]).any(axis=1) | (sc_h[rows] != ref_sc[tok]).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first rows {rows[bad[:8]]} (tokens {tok[bad[:8]]})"
    pads = np.nonzero(got["row_src"][:got["expert_offsets"][-1]] < 0)[0]
    assert not q_h[pads].any() and not sc_h[pads].any()
    g = np.random.default_rng(wid)
    sample = g.choice(rows, 256, replace=False)
    v = values(host(xp)[sample])
    deq = oracle.mx_dequantize(q_h[sample], sc_h[sample])
    s = np.repeat(sc_h[sample].astype(np.int64) - 127, 32, axis=1)
    a = np.abs(v) / 2.0 ** s
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    bound = np.where(a > 448, np.abs(v) - 448 * 2.0 ** s, 2.0 ** (s + e - 4))
    assert (np.abs(deq - v) <= bound).all()


# ------------------------------------------------------------ MXFP8 expert FFN

@pytest.mark.parametrize("rows,cols", [(1, 32), (300, 7168), (1024, 4096), (77, 544)])
def test_mx_quantize(moe, rows, cols):
    g = np.random.default_rng(rows + cols)
    x = mi.f32_to_bf16_bits((g.standard_normal((rows, cols)) * np.exp(g.uniform(-10, 10, (rows, 1)))).astype(np.float32))
    x[0, :32] = 0
    q, s = moe.moe_mx_quantize(dev(x))
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.mx_quantize(x)
    np.testing.assert_array_equal(host(s), ref_s)
    np.testing.assert_array_equal(host(q), ref_q)


def test_mx_quantize_every_value_at_every_scale(moe):
    """The device encoder against the oracle for every bf16 value within 20
    binades below a block maximum, at every scale code (about 1.4 M elements)."""
    x = every_value_at_every_scale()
    q, s = moe.moe_mx_quantize(dev(x))
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.mx_quantize(x)
    np.testing.assert_array_equal(host(s), ref_s)
    np.testing.assert_array_equal(host(q), ref_q)


def mx_ffn_case(moe, w, n_sample, seed=0, experts=None, capacity=0, row_align=0, logits=None):
    """Route, MXFP8 dispatch and MXFP8 FFN on the GPU; the oracle on sampled rows
    of the given experts (its own layout, dispatch and weight quantisation)."""
    if logits is None:
        logits = mi.router_logits(w, seed)
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    e, h, inter, k = w.n_experts, w.hidden, w.inter, w.top_k
    idx, wts, _, _ = oracle.route(logits, k)
    q, sc, _, lay = moe.moe_dispatch_mxfp8(dev(x), dev(idx), dev(wts), e, capacity=capacity, row_align=row_align)
    gq, gs = moe.moe_mx_quantize(dev(wgu))
    dq, ds = moe.moe_mx_quantize(dev(wd))
    y = moe.moe_expert_ffn_mxfp8(q, sc, lay, gq, gs, dq, ds)
    torch.cuda.synchronize()
    ref_lay = oracle.layout(idx, e, capacity, 0, row_align)
    # rows of an unused dropless tail are not written: the oracle keeps what the GPU left there
    ref_q, ref_s, _ = oracle.dispatch_mxfp8(x, k, ref_lay, wts, x_perm_q=host(q).copy(), x_perm_scale=host(sc).copy())
    np.testing.assert_array_equal(host(q), ref_q)
    np.testing.assert_array_equal(host(sc), ref_s)
    g = np.random.default_rng(seed + 1)
    if experts is None:
        experts = np.nonzero(ref_lay["tokens_per_expert"] > 0)[0]
    cand = np.concatenate([np.arange(ref_lay["expert_offsets"][x_], ref_lay["expert_offsets"][x_]
                                     + ref_lay["tokens_per_expert"][x_]) for x_ in experts])
    rows = np.sort(g.choice(cand, min(n_sample, cand.size), replace=False))
    # the weights of the sampled rows' experts, quantised by the oracle (checked against the GPU's)
    rq_gu = np.zeros((e, 2 * inter, h), np.uint8); rs_gu = np.zeros((e, 2 * inter, h // 32), np.uint8)
    rq_d = np.zeros((e, h, inter), np.uint8); rs_d = np.zeros((e, h, inter // 32), np.uint8)
    for x_ in experts:
        rq_gu[x_], rs_gu[x_] = oracle.mx_quantize(wgu[x_])
        rq_d[x_], rs_d[x_] = oracle.mx_quantize(wd[x_])
        np.testing.assert_array_equal(host(gq[x_]), rq_gu[x_])
        np.testing.assert_array_equal(host(gs[x_]), rs_gu[x_])
        np.testing.assert_array_equal(host(dq[x_]), rq_d[x_])
        np.testing.assert_array_equal(host(ds[x_]), rs_d[x_])
    ref_y, ex = oracle.expert_ffn_mxfp8_rows(rows, ref_q, ref_s, ref_lay, rq_gu, rs_gu, rq_d, rs_d)
    assert (ex >= 0).all()
    got = host(y)[rows]
    err = max_rel_err(got, ref_y)
    assert err <= TOL_BF16, err
    return err


def test_mx_ffn_small_ragged(moe):
    """Several experts with ragged last tiles (2 tiles of 512 features, 2 K groups)."""
    w = mi.workload(4, n_tokens=400, hidden=512, n_experts=8, top_k=2, inter=512)
    mx_ffn_case(moe, w, 96)


def test_mx_ffn_qwen3_layer_sampled(moe):
    """The Qwen3-like layer (H=4096, I=1536): sampled rows of three experts."""
    w = mi.workload(4)
    mx_ffn_case(moe, w, 12, experts=[0, 57, 127])


def test_mx_ffn_dsv3_shape_sampled(moe):
    """H=7168, I=2048 (the DeepSeek-like expert shape): 32 experts, top-8 routing."""
    w = mi.workload(4, n_tokens=2048, hidden=7168, n_experts=32, top_k=8, inter=2048)
    mx_ffn_case(moe, w, 8, experts=[3, 30])


@pytest.mark.parametrize("capacity,row_align", [(96, 0), (128, 32), (0, 32), (0, 256)])
def test_mx_ffn_capacity_and_aligned_segments(moe, capacity, row_align):
    """Capacity segments with zero pad rows, and alignment-padded dropless
    segments (the FP8 padding of the routing maps): the pads are all-zero MXFP8
    rows and the FFN computes the kept rows only."""
    w = mi.workload(4, n_tokens=512, hidden=512, n_experts=8, top_k=2, inter=512)
    logits = mi.router_logits(w) + np.log(np.arange(1, 9) ** -1.0).astype(np.float32)  # uneven loads
    mx_ffn_case(moe, w, 64, capacity=capacity, row_align=row_align, logits=logits.astype(np.float32))


def test_mx_ffn_many_experts(moe):
    """1024 experts with a few rows each (most m-tiles ragged, many experts empty)."""
    w = mi.workload(4, n_tokens=600, hidden=512, n_experts=1024, top_k=4, inter=512)
    mx_ffn_case(moe, w, 24, experts=[0, 511, 1023])


def test_mx_ffn_empty_and_empty_experts(moe):
    w = mi.workload(4, n_tokens=64, hidden=512, n_experts=16, top_k=1, inter=512)
    logits = mi.router_logits(w)
    logits[:, 8:] -= 100.0                                 # experts 8..15 receive nothing
    x = mi.activations(w)
    idx, wts, _, _ = oracle.route(logits, 1)
    q, sc, _, lay = moe.moe_dispatch_mxfp8(dev(x), dev(idx), dev(wts), 16)
    wgu, wd = mi.expert_weights(w)
    gq, gs = moe.moe_mx_quantize(dev(wgu))
    dq, ds = moe.moe_mx_quantize(dev(wd))
    y = moe.moe_expert_ffn_mxfp8(q, sc, lay, gq, gs, dq, ds)
    torch.cuda.synchronize()
    assert np.isfinite(mi.bf16_bits_to_f32(host(y))).all()                # every row is kept (top-1, dropless)
    q0, s0, _, lay0 = moe.moe_dispatch_mxfp8(dev(x[:0]), dev(idx[:0]), dev(wts[:0]), 16)
    y0 = moe.moe_expert_ffn_mxfp8(q0, s0, lay0, gq, gs, dq, ds)
    torch.cuda.synchronize()
    assert y0.numel() == 0


def test_mxfp8_and_replicated_steps_replay_in_a_hip_graph(moe):
    """route -> MXFP8 dispatch -> MXFP8 FFN -> combine, and route -> replica plan
    -> weight sync -> reroute -> dispatch -> FFN with replica slots -> combine,
    each captured once in a HIP graph and replayed three times with other work in
    between: every replay equals the eager step bit for bit (the new entry points
    launch kernels only)."""
    n, e, k, h, inter, r_ = 512, 16, 4, 512, 512, 3
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter)
    logits = dev((mi.router_logits(w) + np.log(np.arange(1, e + 1) ** -1.5).astype(np.float32) * 3).astype(np.float32))
    x = dev(mi.activations(w))
    wgu, wd = (dev(a) for a in mi.expert_weights(w))
    gq, gs = moe.moe_mx_quantize(wgu)
    dq, ds = moe.moe_mx_quantize(wd)
    rt = moe.moe_route(logits, k)
    q8, s8, _, lay8 = moe.moe_dispatch_mxfp8(x, rt.topk_idx, rt.topk_w, e)
    y8 = torch.empty((lay8.rows, h), dtype=torch.bfloat16, device="cuda")
    out8 = torch.empty_like(x)
    rep = moe.moe_replica_plan(rt.tokens_per_expert, r_)
    wgu_r, wd_r = moe.moe_replica_sync(wgu, wd, rep)
    phys = moe.moe_reroute(rt.topk_idx, e, rep)
    xp, wp, lay = moe.moe_dispatch(x, phys, rt.topk_w, e + r_)
    y = torch.empty_like(xp)
    out = torch.empty_like(x)
    ws_d = moe.alloc_workspace(moe.MOE_OP_DISPATCH, moe.make_shape(n, h, e + r_, k), "cuda")
    ws_8 = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN_MXFP8, lay8.shape(h, moe.MOE_DT_BF16, inter), "cuda")
    ws_f = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN, lay.shape(h, moe.MOE_DT_BF16, inter), "cuda")
    ws_r = moe.alloc_workspace(moe.MOE_OP_REROUTE, moe.make_shape(n, 1, e, k), "cuda")

    def step():
        moe.moe_route(logits, k, out=rt)
        moe.moe_dispatch_mxfp8(x, rt.topk_idx, rt.topk_w, e, layout=lay8, x_perm_q=q8, x_perm_scale=s8,
                               w_perm=False, workspace=ws_d)
        moe.moe_expert_ffn_mxfp8(q8, s8, lay8, gq, gs, dq, ds, y=y8, workspace=ws_8)
        moe.moe_combine(y8, rt.topk_w, lay8, out=out8)
        moe.moe_replica_plan(rt.tokens_per_expert, r_, out=rep)
        moe.moe_replica_sync(wgu, wd, rep, w_gate_up_replica=wgu_r, w_down_replica=wd_r)
        moe.moe_reroute(rt.topk_idx, e, rep, out=phys, workspace=ws_r)
        moe.moe_dispatch(x, phys, rt.topk_w, e + r_, layout=lay, x_perm=xp, w_perm_out=wp, workspace=ws_d)
        moe.moe_expert_ffn_replicas(xp, lay, wgu, wd, wgu_r, wd_r, y=y, workspace=ws_f)
        moe.moe_combine(y, rt.topk_w, lay, out=out)

    step()
    torch.cuda.synchronize()
    ref8, ref, ref_phys = out8.clone(), out.clone(), phys.clone()
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
    for _ in range(3):
        out8.fill_(7.0)
        out.fill_(7.0)
        phys.fill_(-5)
        q8.fill_(0)
        torch.randn(1 << 20, device="cuda").sum()           # other work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out8, ref8) and torch.equal(out, ref) and torch.equal(phys, ref_phys)
    del g
