"""Randomised GPU parity sweep through the C ABI: 24 seeded draws of the shape
and options of a layer (tokens, experts, top-k, hidden size, capacity, drop
policy, alignment, row budget, sentinel and invalid ids), each checked bit for
bit against the CPU oracle for routing, layout, dispatched rows (bf16 and
MXFP8), the combine's fp32 accumulation and the dispatch backward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_F32, assert_layout_equal, dev, host, layout_host, max_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def draw(seed):
    g = np.random.default_rng(9000 + seed)
    n = int(g.choice([0, 1, 7, 130, 777, 2049]))
    e = int(g.choice([1, 3, 16, 64, 200, 1024]))
    k = int(min(e, g.choice([1, 2, 3, 8])))
    h = int(g.choice([32, 96, 512, 1056]))
    cap = int(g.choice([0, 0, 1, 5, 40])) if seed % 3 else 0
    align = int(g.choice([0, 1, 4, 32])) if cap == 0 else 0
    policy = int(g.integers(0, 2)) if cap else 0
    budget = int(max(0, n * k - g.integers(0, 50))) if (cap == 0 and seed % 5 == 0 and n) else 0
    return g, n, e, k, h, cap, align, policy, budget


@pytest.mark.parametrize("seed", range(24))
def test_random_layer(moe, seed):
    g, n, e, k, h, cap, align, policy, budget = draw(seed)
    logits = g.standard_normal((n, e)).astype(np.float32)
    if seed % 4 == 1:
        logits = np.round(logits * 2) / 2                       # many ties
    r = moe.moe_route(dev(logits), k)
    torch.cuda.synchronize()
    idx, wts, rmap, tpe = oracle.route(logits, k)
    np.testing.assert_array_equal(host(r.topk_idx), idx)
    np.testing.assert_array_equal(host(r.tokens_per_expert), tpe)
    if n:
        assert max_rel_err(host(r.topk_w), wts) <= TOL_F32
    # sentinels and invalid ids on the dispatch side
    idx2 = idx.copy()
    if n and seed % 2:
        idx2[g.random(idx2.shape) < 0.1] = -1
        idx2[g.random(idx2.shape) < 0.03] = g.choice([-4, e, e + 7])
    x = mi.f32_to_bf16_bits(g.standard_normal((n, h)).astype(np.float32))
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx2), dev(wts), e, capacity=cap, max_rows=budget, row_align=align,
                                   drop_policy=policy)
    q8, s8, wp8, lay8 = moe.moe_dispatch_mxfp8(dev(x), dev(idx2), dev(wts), e, capacity=cap, max_rows=budget,
                                               row_align=align, drop_policy=policy)
    torch.cuda.synchronize()
    ref = oracle.layout(idx2, e, cap, budget, align, policy, wts)
    assert_layout_equal(layout_host(lay), ref)
    assert_layout_equal(layout_host(lay8), ref)
    xp_h = host(xp)
    ref_xp, ref_wp = oracle.scatter(x, k, ref, wts, x_perm=xp_h.copy())
    assert (xp_h.view(np.uint8) == ref_xp.view(np.uint8)).all()
    np.testing.assert_array_equal(host(wp), ref_wp)
    rq, rs, _ = oracle.dispatch_mxfp8(x, k, ref, wts, x_perm_q=host(q8).copy(), x_perm_scale=host(s8).copy())
    np.testing.assert_array_equal(host(q8), rq)
    np.testing.assert_array_equal(host(s8), rs)
    # identity expert: the combine's fp32 slot-order accumulation and the dispatch backward
    out = moe.moe_combine(xp, dev(wts), lay)
    gx = moe.moe_dispatch_bwd(xp, lay)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), oracle.combine(xp_h, wts, ref, n, k))
    np.testing.assert_array_equal(host(gx), oracle.dispatch_bwd(xp_h, ref, n, k))
