"""Seeded random draws of the expert FFN forward and backward through the C ABI, against the oracle.

Each draw picks the expert count (1-23), hidden size (64-640) and intermediate size
(64-512, multiples of 64, so most weight gradients have ragged edge tiles in both
dimensions) and a row-count pattern: uniform 0-699 rows per expert, one heavy
expert of 1000-4000 rows over light ones (a unit the weight gradients' work plan
splits into parts, whose tiles run in chains of two), or Zipf-distributed counts.
Rows go to experts with one slot per token.  The forward stores the
pre-activations, the backward takes them; the output on every kept row and on
every expert's segment, dX on every segment row, dW_gate_up and dW_down of every
expert (and of every 256 x 256 tile of them on its own) must meet the bf16
tolerance, and experts without rows must get zero gradients."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_BF16, dev, host, layout_host, max_rel_err


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def draw(rng):
    e = int(rng.integers(1, 24))
    h = int(rng.integers(1, 11)) * 64
    inter = int(rng.integers(1, 9)) * 64
    kind = int(rng.integers(0, 3))
    if kind == 0:
        counts = rng.integers(0, 700, e)
    elif kind == 1:
        counts = np.zeros(e, np.int64)
        counts[rng.integers(0, e)] = int(rng.integers(1000, 4000))
        counts += rng.integers(0, 40, e) * (rng.random(e) < 0.5)
    else:
        counts = (rng.zipf(1.3, e) * 37) % 2500
    counts = counts.astype(np.int64)
    if counts.sum() == 0:
        counts[0] = 1
    return e, h, inter, counts


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(12))
def test_ffn_random_draw(moe, seed):
    e, h, inter, counts = draw(np.random.default_rng(1000 + seed))
    n = int(counts.sum())
    print(f"seed {seed}: e={e} h={h} inter={inter} counts={counts.tolist()}", flush=True)
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=1, inter=inter)
    idx = np.repeat(np.arange(e, dtype=np.int32), counts).reshape(n, 1)
    wts = np.ones((n, 1), np.float32)
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e)
    y, gu = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd), save_gate_up=True)
    dy = mi.grad_expert_rows(w, lay.rows, seed)
    gx, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, dev(dy), lay, dev(wgu), dev(wd), gate_up=gu)
    torch.cuda.synchronize()
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    np.testing.assert_array_equal(lay_h["tokens_per_expert"], counts.astype(np.int32))
    ref_y = oracle.expert_ffn(host(xp), lay_h, wgu, wd)
    kept = lay_h["pad_mask"] == 0
    assert max_rel_err(host(y)[kept], ref_y[kept]) <= TOL_BF16
    ref_gx, ref_dwgu, ref_dwd = oracle.expert_ffn_bwd(host(xp), dy, lay_h, wgu, wd)
    gx_h, dwgu_h, dwd_h = host(gx), host(dwgu), host(dwd)
    offs = lay_h["expert_offsets"]
    for ex, c in enumerate(counts):
        if not c:
            assert not dwgu_h[ex].any() and not dwd_h[ex].any(), ex
            continue
        seg = slice(offs[ex], offs[ex] + c)
        assert max_rel_err(host(y)[seg], ref_y[seg]) <= TOL_BF16, (ex, int(c))
        errs = (max_rel_err(gx_h[seg], ref_gx[seg]), max_rel_err(dwgu_h[ex], ref_dwgu[ex]),
                max_rel_err(dwd_h[ex], ref_dwd[ex]))
        assert max(errs) <= TOL_BF16, (ex, int(c), errs)
        for g, r in ((dwgu_h[ex], ref_dwgu[ex]), (dwd_h[ex], ref_dwd[ex])):
            for m0 in range(0, g.shape[0], 256):
                for n0 in range(0, g.shape[1], 256):
                    t = (slice(m0, m0 + 256), slice(n0, n0 + 256))
                    assert max_rel_err(g[t], r[t]) <= TOL_BF16, (ex, int(c), g.shape, m0, n0)
