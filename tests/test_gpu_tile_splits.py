"""The grouped GEMM's m-tiles at every split the tile lookup makes, through the C ABI.

An expert's rows are split evenly over its ceil(rows / 256) m-tiles in whole
32-row blocks, and each wave runs the MFMAs of the one to four row blocks it
holds.  Experts here get row counts chosen so that every such case occurs:
one tile of 1, 31-33, 64-65, 96, 160, 192, 224 and 255-256 rows (each wave
holding 0-4 blocks, the two wave rows holding different counts), two tiles
(257: 160 + 97, 300, 384: 192 + 192, 385: 224 + 161, 448, 512), three tiles
(513: 192 + 192 + 129, 520, 640, 768), four tiles (769, 1000) and an expert
without rows.  The bf16 forward (every row) and backward (every segment row
of dX, every weight gradient) are compared with the oracle, and the MXFP8
forward on rows at the edges of every m-tile of a subset of the experts (the
first and last row of each tile and of its first two 32-row blocks, and its
middle row).  Routing is one slot per token, token t to the expert whose
cumulative count covers t."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import TOL_BF16, dev, host, layout_host, max_rel_err

COUNTS = [1, 31, 32, 33, 64, 65, 96, 160, 192, 224, 255, 256, 257, 300, 384, 385, 448, 512, 0, 513, 520, 640,
          768, 769, 1000]


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def split_case(counts, h, inter, seed):
    """Inputs whose layout gives expert x exactly counts[x] rows (k = 1)."""
    e, n = len(counts), int(sum(counts))
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=1, inter=inter)
    idx = np.repeat(np.arange(e, dtype=np.int32), counts).reshape(n, 1)
    wts = np.ones((n, 1), np.float32)
    x = mi.activations(w, seed)
    wgu, wd = mi.expert_weights(w, seed)
    return w, idx, wts, x, wgu, wd


def tile_edge_rows(count):
    """Rows (relative to the expert's segment) at the edges of its m-tiles under
    the even split: ceil(count / 256) tiles of q 32-row blocks, the last fewer."""
    tiles = (count + 255) // 256
    q = ((count + 31) // 32 + tiles - 1) // tiles
    out = set()
    for m in range(tiles):
        first, last = m * q * 32, min((m + 1) * q * 32, count) - 1
        for r in (first, first + 31, first + 32, first + 63, (first + last) // 2, last):
            if first <= r <= last:
                out.add(r)
    return sorted(out)


def test_tile_edge_rows_cover_every_tile():
    """The sampled rows touch every tile, and the tiles cover the segment."""
    for c in range(1, 3000):
        tiles = (c + 255) // 256
        q = ((c + 31) // 32 + tiles - 1) // tiles
        assert q <= 8 and (tiles - 1) * q * 32 < c <= tiles * q * 32
        rows = tile_edge_rows(c)
        assert rows[0] == 0 and rows[-1] == c - 1
        assert len({r // (q * 32) for r in rows}) == tiles


@pytest.mark.gpu
def test_tile_splits_bf16_forward_and_backward(moe):
    w, idx, wts, x, wgu, wd = split_case(COUNTS, 256, 128, 5)
    e = w.n_experts
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e)
    y = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd))
    dy = mi.grad_expert_rows(w, lay.rows, 5)
    gx, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, dev(dy), lay, dev(wgu), dev(wd))
    torch.cuda.synchronize()
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    np.testing.assert_array_equal(lay_h["tokens_per_expert"], np.asarray(COUNTS, np.int32))
    kept = lay_h["pad_mask"] == 0
    ref = oracle.expert_ffn(host(xp), lay_h, wgu, wd)
    got = host(y)
    assert max_rel_err(got[kept], ref[kept]) <= TOL_BF16
    assert (got[kept] == ref[kept]).mean() > 0.9
    # the worst expert too, so that one bad tile cannot hide behind the others' scale
    offs = lay_h["expert_offsets"]
    for ex, c in enumerate(COUNTS):
        if c:
            seg = slice(offs[ex], offs[ex] + c)
            assert max_rel_err(got[seg], ref[seg]) <= TOL_BF16, (ex, c)
    ref_gx, ref_dwgu, ref_dwd = oracle.expert_ffn_bwd(host(xp), dy, lay_h, wgu, wd)
    gx_h, dwgu_h, dwd_h = host(gx), host(dwgu), host(dwd)
    for ex, c in enumerate(COUNTS):
        if c:
            seg = slice(offs[ex], offs[ex] + c)
            errs = (max_rel_err(gx_h[seg], ref_gx[seg]), max_rel_err(dwgu_h[ex], ref_dwgu[ex]),
                    max_rel_err(dwd_h[ex], ref_dwd[ex]))
            assert max(errs) <= TOL_BF16, (ex, c, errs)
        else:
            assert not dwgu_h[ex].any() and not dwd_h[ex].any()


# Weight gradients run their output tiles in chains: workgroup c of a unit of T
# tiles (a whole expert, or a part of a heavy one) runs tiles c and c + C with
# C = ceil(T / 2), the load ring running on across the two.  H = 576 and
# I = 192 make ragged edge tiles in both output dimensions of both gradients
# (dW_gate_up 384 x 576: 2 x 3 tiles; dW_down 576 x 192: 3 x 1 tiles, so one
# chain of a single tile), so a chain joins tiles with different edge clamps;
# the 2000-row expert holds more than 1/16 of all K steps and is split into
# parts, some with no tile, and so are the 300- and 513-row experts; expert 0
# has no rows.
CHAIN_COUNTS = [0, 1, 65, 300, 2000, 70, 129, 513]


@pytest.mark.gpu
def test_weight_gradient_chains(moe):
    w, idx, wts, x, wgu, wd = split_case(CHAIN_COUNTS, 576, 192, 7)
    e = w.n_experts
    xp, wp, lay = moe.moe_dispatch(dev(x), dev(idx), dev(wts), e)
    y, gu = moe.moe_expert_ffn(xp, lay, dev(wgu), dev(wd), save_gate_up=True)
    dy = mi.grad_expert_rows(w, lay.rows, 7)
    gx, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, dev(dy), lay, dev(wgu), dev(wd), gate_up=gu)
    torch.cuda.synchronize()
    lay_h = layout_host(lay)
    lay_h["rows"] = lay.rows
    np.testing.assert_array_equal(lay_h["tokens_per_expert"], np.asarray(CHAIN_COUNTS, np.int32))
    ref_gx, ref_dwgu, ref_dwd = oracle.expert_ffn_bwd(host(xp), dy, lay_h, wgu, wd)
    gx_h, dwgu_h, dwd_h = host(gx), host(dwgu), host(dwd)
    offs = lay_h["expert_offsets"]
    for ex, c in enumerate(CHAIN_COUNTS):
        if c:
            seg = slice(offs[ex], offs[ex] + c)
            errs = (max_rel_err(gx_h[seg], ref_gx[seg]), max_rel_err(dwgu_h[ex], ref_dwgu[ex]),
                    max_rel_err(dwd_h[ex], ref_dwd[ex]))
            assert max(errs) <= TOL_BF16, (ex, c, errs)
            # every 256 x 256 tile of both gradients on its own, edge tiles included
            for g, r in ((dwgu_h[ex], ref_dwgu[ex]), (dwd_h[ex], ref_dwd[ex])):
                for m0 in range(0, g.shape[0], 256):
                    for n0 in range(0, g.shape[1], 256):
                        t = (slice(m0, m0 + 256), slice(n0, n0 + 256))
                        assert max_rel_err(g[t], r[t]) <= TOL_BF16, (ex, c, g.shape, m0, n0)
        else:
            assert not dwgu_h[ex].any() and not dwd_h[ex].any()


@pytest.mark.gpu
def test_tile_splits_mxfp8_forward(moe):
    counts = [33, 96, 160, 224, 257, 385, 513, 769]
    w, idx, wts, x, wgu, wd = split_case(counts, 512, 512, 6)
    e, h, inter = w.n_experts, w.hidden, w.inter
    q, sc, _, lay = moe.moe_dispatch_mxfp8(dev(x), dev(idx), dev(wts), e)
    gq, gs = moe.moe_mx_quantize(dev(wgu))
    dq, ds = moe.moe_mx_quantize(dev(wd))
    y = moe.moe_expert_ffn_mxfp8(q, sc, lay, gq, gs, dq, ds)
    torch.cuda.synchronize()
    ref_lay = oracle.layout(idx, e, 0, 0)
    np.testing.assert_array_equal(ref_lay["tokens_per_expert"], np.asarray(counts, np.int32))
    ref_q, ref_s, _ = oracle.dispatch_mxfp8(x, 1, ref_lay, wts, x_perm_q=host(q).copy(), x_perm_scale=host(sc).copy())
    np.testing.assert_array_equal(host(q), ref_q)
    rq_gu = np.zeros((e, 2 * inter, h), np.uint8); rs_gu = np.zeros((e, 2 * inter, h // 32), np.uint8)
    rq_d = np.zeros((e, h, inter), np.uint8); rs_d = np.zeros((e, h, inter // 32), np.uint8)
    for x_ in range(e):
        rq_gu[x_], rs_gu[x_] = oracle.mx_quantize(wgu[x_])
        rq_d[x_], rs_d[x_] = oracle.mx_quantize(wd[x_])
    offs = ref_lay["expert_offsets"]
    per = [np.asarray(tile_edge_rows(c)) + offs[x_] for x_, c in enumerate(counts)]
    rows = np.concatenate(per)
    ref_y, ex = oracle.expert_ffn_mxfp8_rows(rows, ref_q, ref_s, ref_lay, rq_gu, rs_gu, rq_d, rs_d)
    got = host(y)[rows]
    at = 0
    for x_, c in enumerate(counts):
        seg = slice(at, at + len(per[x_]))
        at += len(per[x_])
        assert (ex[seg] == x_).all()
        assert max_rel_err(got[seg], ref_y[seg]) <= TOL_BF16, (x_, c)
