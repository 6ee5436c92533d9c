"""GPU parity of the hot-expert replication calls against the CPU oracle, through
the C ABI: placement, reroute and weight sync bit-exact; the gradient reduce
bit-exact on data whose sums are exact and within the bf16 tolerance otherwise;
the grouped FFN with replica weight slots bit for bit equal to the same FFN over
one weight tensor holding masters and replicas; and a replicated layer
(route -> plan -> sync -> reroute -> dispatch -> FFN -> combine) equal bit for
bit to the unreplicated one, its backward within tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_BF16, dev, host, max_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


@pytest.mark.parametrize("e,r,kind", [(8, 0, "random"), (8, 5, "random"), (256, 16, "random"), (1000, 24, "random"),
                                      (64, 300, "random"), (16, 7, "equal"), (32, 9, "zeros"), (1024, 1024, "random"),
                                      (5, 40, "one_hot")])
def test_replica_plan(moe, e, r, kind):
    g = np.random.default_rng(e * 7 + r)
    counts = (g.zipf(1.5, e) * 13 % 5000).astype(np.int32)
    if kind == "equal":
        counts[:] = 77
    if kind == "zeros":
        counts[:] = 0
    if kind == "one_hot":
        counts[:] = 0
        counts[3] = 1000
    got = moe.moe_replica_plan(dev(counts), r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), oracle.replica_plan(counts, r))


@pytest.mark.parametrize("n,e,k,r", [(1000, 16, 4, 4), (4096, 256, 8, 16), (333, 7, 7, 20), (64, 1, 1, 3),
                                     (2048, 128, 8, 128)])
def test_reroute(moe, n, e, k, r):
    g = np.random.default_rng(n + e + k + r)
    bias = np.log(np.arange(1, e + 1, dtype=np.float64) ** -1.2) * 2
    logits = (g.standard_normal((n, e)) + bias).astype(np.float32)
    idx, _, _, counts = oracle.route(logits, k)
    if n > 500:                                           # sentinels and invalid ids
        idx[g.random(idx.shape) < 0.05] = -1
        idx[g.random(idx.shape) < 0.02] = g.choice([-3, e, e + 9])
        counts = np.bincount(idx[(idx >= 0) & (idx < e)], minlength=e).astype(np.int32)
    rep = oracle.replica_plan(counts, r)
    got = moe.moe_reroute(dev(idx), e, dev(rep))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), oracle.reroute(idx, e, rep))
    # in place
    buf = dev(idx)
    moe.moe_reroute(buf, e, dev(rep), out=buf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(buf), oracle.reroute(idx, e, rep))


def test_reroute_empty(moe):
    idx = np.zeros((0, 4), np.int32)
    got = moe.moe_reroute(dev(idx), 8, dev(np.array([1, 2], np.int32)))
    torch.cuda.synchronize()
    assert got.numel() == 0


def test_replica_sync_and_grad_reduce(moe):
    e, h, inter = 6, 128, 64
    rep = np.array([2, 4, 2, 0, 2], np.int32)
    g = np.random.default_rng(9)
    wgu = mi.f32_to_bf16_bits(g.standard_normal((e, 2 * inter, h)).astype(np.float32))
    wd = mi.f32_to_bf16_bits(g.standard_normal((e, h, inter)).astype(np.float32))
    a, b = moe.moe_replica_sync(dev(wgu), dev(wd), dev(rep))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a), oracle.replica_sync(wgu, rep))
    np.testing.assert_array_equal(host(b), oracle.replica_sync(wd, rep))
    # a slot naming no expert is skipped: its buffer keeps what it held
    bad = np.array([1, 77, -1], np.int32)
    a2 = torch.full((3, 2 * inter, h), 3.0, dtype=torch.bfloat16, device="cuda")
    b2 = torch.full((3, h, inter), 3.0, dtype=torch.bfloat16, device="cuda")
    moe.moe_replica_sync(dev(wgu), dev(wd), dev(bad), w_gate_up_replica=a2, w_down_replica=b2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(a2)[0], wgu[1])
    assert (a2[1:].float() == 3.0).all() and (b2[1:].float() == 3.0).all()
    # reduce: small integers (every sum exact: bit-exact), then general values (tolerance)
    for ints in (True, False):
        if ints:
            gm = [g.integers(-60, 60, s).astype(np.float32) for s in ((e, 2 * inter, h), (e, h, inter))]
            gr = [g.integers(-60, 60, s).astype(np.float32) for s in ((5, 2 * inter, h), (5, h, inter))]
        else:
            gm = [g.standard_normal(s).astype(np.float32) for s in ((e, 2 * inter, h), (e, h, inter))]
            gr = [g.standard_normal(s).astype(np.float32) for s in ((5, 2 * inter, h), (5, h, inter))]
        gm = [mi.f32_to_bf16_bits(t) for t in gm]
        gr = [mi.f32_to_bf16_bits(t) for t in gr]
        d_gm = [dev(t) for t in gm]
        moe.moe_replica_grad_reduce(d_gm[0], d_gm[1], dev(gr[0]), dev(gr[1]), dev(rep))
        torch.cuda.synchronize()
        for got, m_, r_ in zip(d_gm, gm, gr):
            want = oracle.replica_grad_reduce(m_, r_, rep)
            if ints:
                np.testing.assert_array_equal(host(got), want)
            else:
                assert max_rel_err(host(got), want) <= TOL_BF16
                assert (host(got) == want).mean() > 0.999
            np.testing.assert_array_equal(host(got)[[1, 3, 5]], m_[[1, 3, 5]])


def replicated_inputs(n=512, e=16, k=4, h=256, inter=128, r=4, seed=0):
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter)
    logits = mi.router_logits(w, seed) + np.log(np.arange(1, e + 1) ** -1.5).astype(np.float32) * 3
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    go = mi.grad_output(w, seed)
    return w, logits.astype(np.float32), x, wgu, wd, go


def test_ffn_replica_slots_equal_one_weight_tensor(moe):
    """Two storage bases give the same bits as one tensor [masters; replicas]."""
    w, logits, x, wgu, wd, go = replicated_inputs()
    e, k, r = w.n_experts, w.top_k, 4
    rt = moe.moe_route(dev(logits), k)
    rep = moe.moe_replica_plan(rt.tokens_per_expert, r)
    wgu_r, wd_r = moe.moe_replica_sync(dev(wgu), dev(wd), rep)
    phys = moe.moe_reroute(rt.topk_idx, e, rep)
    xp, wp, lay = moe.moe_dispatch(dev(x), phys, rt.topk_w, e + r)
    y1, gu1 = moe.moe_expert_ffn_replicas(xp, lay, dev(wgu), dev(wd), wgu_r, wd_r, save_gate_up=True)
    cat_gu, cat_d = torch.cat([dev(wgu), wgu_r]), torch.cat([dev(wd), wd_r])
    y2, gu2 = moe.moe_expert_ffn(xp, lay, cat_gu, cat_d, save_gate_up=True)
    gy = torch.randn(xp.shape, generator=torch.Generator(device="cuda").manual_seed(3), device="cuda").bfloat16()
    b1 = moe.moe_expert_ffn_bwd_replicas(xp, gy, lay, dev(wgu), dev(wd), wgu_r, wd_r, gate_up=gu1)
    b2 = moe.moe_expert_ffn_bwd(xp, gy, lay, cat_gu, cat_d, gate_up=gu2)
    torch.cuda.synchronize()
    kept = torch.from_numpy(host(lay.pad_mask) == 0).cuda()
    assert torch.equal(y1[kept], y2[kept]) and torch.equal(gu1[kept], gu2[kept])
    assert torch.equal(b1[0][kept], b2[0][kept])
    assert torch.equal(b1[1], b2[1][:e]) and torch.equal(b1[3], b2[1][e:])
    assert torch.equal(b1[2], b2[2][:e]) and torch.equal(b1[4], b2[2][e:])
    # and against the oracle
    ref_y = oracle.expert_ffn(host(xp), {f: host(getattr(lay, f)) for f in ("tokens_per_expert", "expert_offsets",
                                                                            "pad_mask", "row_src")} | {"rows": lay.rows},
                              host(cat_gu), host(cat_d))
    kh = host(lay.pad_mask) == 0
    assert max_rel_err(host(y1)[kh], ref_y[kh]) <= TOL_BF16


@pytest.mark.parametrize("r", [1, 4, 13])
def test_replicated_layer_matches_unreplicated(moe, r):
    """The expert rows of a token do not depend on which copy computes them, so
    the replicated layer's output is the unreplicated one bit for bit; the
    backward's token gradients too, and the reduced weight gradients agree with
    the unreplicated ones within tolerance (their sums are split differently)."""
    w, logits, x, wgu, wd, go = replicated_inputs(seed=r)
    e, k = w.n_experts, w.top_k
    rt = moe.moe_route(dev(logits), k)
    # unreplicated
    xp0, _, lay0 = moe.moe_dispatch(dev(x), rt.topk_idx, rt.topk_w, e)
    y0, gu0 = moe.moe_expert_ffn(xp0, lay0, dev(wgu), dev(wd), save_gate_up=True)
    out0 = moe.moe_combine(y0, rt.topk_w, lay0)
    gy0, gw0 = moe.moe_combine_bwd(dev(go), y0, rt.topk_w, lay0)
    gxp0, dwgu0, dwd0 = moe.moe_expert_ffn_bwd(xp0, gy0, lay0, dev(wgu), dev(wd), gate_up=gu0)
    gx0 = moe.moe_dispatch_bwd(gxp0, lay0)
    # replicated
    rep = moe.moe_replica_plan(rt.tokens_per_expert, r)
    wgu_r, wd_r = moe.moe_replica_sync(dev(wgu), dev(wd), rep)
    phys = moe.moe_reroute(rt.topk_idx, e, rep)
    xp1, _, lay1 = moe.moe_dispatch(dev(x), phys, rt.topk_w, e + r)
    y1, gu1 = moe.moe_expert_ffn_replicas(xp1, lay1, dev(wgu), dev(wd), wgu_r, wd_r, save_gate_up=True)
    out1 = moe.moe_combine(y1, rt.topk_w, lay1)
    gy1, gw1 = moe.moe_combine_bwd(dev(go), y1, rt.topk_w, lay1)
    gxp1, dwgu1, dwd1, dwgu_r, dwd_r = moe.moe_expert_ffn_bwd_replicas(xp1, gy1, lay1, dev(wgu), dev(wd), wgu_r, wd_r,
                                                                       gate_up=gu1)
    moe.moe_replica_grad_reduce(dwgu1, dwd1, dwgu_r, dwd_r, rep)
    gx1 = moe.moe_dispatch_bwd(gxp1, lay1)
    torch.cuda.synchronize()
    rep_h = host(rep)
    counts = host(rt.tokens_per_expert)
    np.testing.assert_array_equal(rep_h, oracle.replica_plan(counts, r))
    phys_ref = oracle.reroute(host(rt.topk_idx), e, rep_h)
    np.testing.assert_array_equal(host(phys), phys_ref)
    # per-copy loads: the physical counts of the rerouted ids, none above the hottest logical load
    tpe1 = host(lay1.tokens_per_expert)
    np.testing.assert_array_equal(tpe1, np.bincount(phys_ref[phys_ref >= 0], minlength=e + r))
    assert tpe1.max() <= counts.max() and tpe1[e:].min() > 0
    assert torch.equal(out1, out0)
    assert torch.equal(gw1, gw0)
    assert torch.equal(gx1, gx0)
    assert max_rel_err(host(dwgu1), host(dwgu0)) <= TOL_BF16
    assert max_rel_err(host(dwd1), host(dwd0)) <= TOL_BF16
    untouched = np.setdiff1d(np.arange(e), rep_h)           # experts without slots: same rows, same sums
    assert torch.equal(dwgu1[untouched], dwgu0[untouched]) and torch.equal(dwd1[untouched], dwd0[untouched])
