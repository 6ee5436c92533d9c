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


def tile_edge_rows(count):
    """Rows (relative to an expert's segment) at the edges of its m-tiles: the
    grouped GEMM splits a segment's 32-row blocks evenly over ceil(count / 256)
    tiles; the first and last row of each tile, of its first two blocks, and its
    middle row."""
    tiles = (count + 255) // 256
    q = ((count + 31) // 32 + tiles - 1) // tiles
    out = set()
    for m in range(tiles):
        first, last = m * q * 32, min((m + 1) * q * 32, count) - 1
        for r in (first, first + 31, first + 32, first + 63, (first + last) // 2, last):
            if first <= r <= last:
                out.add(r)
    return sorted(out)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(6))
def test_ffn_mxfp8_random_draw(moe, seed):
    """The MXFP8 FFN (rows quantised by the MXFP8 dispatch, weights by
    moe_mx_quantize) on random expert counts, sizes (hidden 512-1536, intermediate
    512 or 1024: whole scale groups) and row counts, against the oracle on every
    tile's edge rows of every expert."""
    rng = np.random.default_rng(2000 + seed)
    e = int(rng.integers(1, 13))
    h = int(rng.integers(1, 4)) * 512
    inter = int(rng.integers(1, 3)) * 512
    counts = rng.integers(0, 900, e).astype(np.int64)
    if counts.sum() == 0:
        counts[0] = 1
    n = int(counts.sum())
    print(f"seed {seed}: e={e} h={h} inter={inter} counts={counts.tolist()}", flush=True)
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=1, inter=inter)
    idx = np.repeat(np.arange(e, dtype=np.int32), counts).reshape(n, 1)
    wts = np.ones((n, 1), np.float32)
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    q, sc, _, lay = moe.moe_dispatch_mxfp8(dev(x), dev(idx), dev(wts), e)
    gq, gs = moe.moe_mx_quantize(dev(wgu))
    dq, ds = moe.moe_mx_quantize(dev(wd))
    y = moe.moe_expert_ffn_mxfp8(q, sc, lay, gq, gs, dq, ds)
    torch.cuda.synchronize()
    ref_lay = oracle.layout(idx, e, 0, 0)
    np.testing.assert_array_equal(ref_lay["tokens_per_expert"], counts.astype(np.int32))
    ref_q, ref_s, _ = oracle.dispatch_mxfp8(x, 1, ref_lay, wts, x_perm_q=host(q).copy(), x_perm_scale=host(sc).copy())
    np.testing.assert_array_equal(host(q), ref_q)
    rq_gu = np.zeros((e, 2 * inter, h), np.uint8); rs_gu = np.zeros((e, 2 * inter, h // 32), np.uint8)
    rq_d = np.zeros((e, h, inter), np.uint8); rs_d = np.zeros((e, h, inter // 32), np.uint8)
    for x_ in range(e):
        rq_gu[x_], rs_gu[x_] = oracle.mx_quantize(wgu[x_])
        rq_d[x_], rs_d[x_] = oracle.mx_quantize(wd[x_])
    np.testing.assert_array_equal(host(gq), rq_gu.reshape(host(gq).shape))
    offs = ref_lay["expert_offsets"]
    per = [np.asarray(tile_edge_rows(int(c)), dtype=np.int64) + offs[x_] for x_, c in enumerate(counts)]
    rows = np.concatenate(per) if per else np.zeros(0, np.int64)
    ref_y, ex = oracle.expert_ffn_mxfp8_rows(rows, ref_q, ref_s, ref_lay, rq_gu, rs_gu, rq_d, rs_d)
    got = host(y)[rows]
    at = 0
    for x_, c in enumerate(counts):
        seg = slice(at, at + len(per[x_]))
        at += len(per[x_])
        assert (ex[seg] == x_).all()
        assert max_rel_err(got[seg], ref_y[seg]) <= TOL_BF16, (x_, int(c))
