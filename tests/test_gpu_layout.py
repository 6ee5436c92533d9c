"""GPU parity of moe_build_layout (the dispatch layout alone) and of the
single-pass look-back scan at sizes where it runs many tiles: every layout
field bit for bit against the CPU oracle, through the C ABI.  Also the scan's
reporting path when its workspace header was not zeroed (forced from the host:
every tile then skips its work, no wait happens, every kernel exits), and the
workspace's reuse across calls of different sizes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_layout_equal, dev, host, layout_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def random_routing(n, e, k, seed, sentinel=0.0):
    """k distinct experts per token (random order), a share of -1 sentinels."""
    g = np.random.default_rng(seed)
    idx = np.argsort(g.random((n, e), dtype=np.float32), axis=1)[:, :k].astype(np.int32)
    if sentinel:
        idx[g.random(idx.shape) < sentinel] = -1
    wts = g.random((n, k), dtype=np.float32)
    return np.ascontiguousarray(idx), wts


@pytest.mark.parametrize("n,e,k,cap,align,policy,sent", [
    (65536, 256, 8, 0, 0, 0, 0.0),      # 524288 assignments: 256 look-back tiles
    (65536, 256, 8, 2560, 0, 0, 0.0),   # the same with a capacity of 1.25x the mean load
    (32768, 1024, 8, 0, 0, 0, 0.1),     # the most experts, sentinels
    (20000, 64, 6, 0, 128, 0, 0.2),     # aligned segments
    (30000, 128, 4, 700, 0, 1, 0.0),    # drop by weight
    (1, 8, 2, 0, 0, 0, 0.0),
])
def test_build_layout_many_tiles(moe, n, e, k, cap, align, policy, sent):
    print(f"build_layout n={n} e={e} k={k} capacity={cap} align={align} policy={policy}", flush=True)
    idx, wts = random_routing(n, e, k, n + e + k, sent)
    wp, lay = moe.moe_build_layout(dev(idx), dev(wts), e, capacity=cap, row_align=align, drop_policy=policy)
    torch.cuda.synchronize()
    ref = oracle.layout(idx, e, cap, 0, align, policy, wts)
    assert_layout_equal(layout_host(lay), ref)
    ref_wp = np.zeros(ref["rows"], np.float32)
    kept = ref["assign_row"] >= 0
    ref_wp[ref["assign_row"][kept]] = wts.reshape(-1)[kept]
    np.testing.assert_array_equal(host(wp), ref_wp)


def test_build_layout_equals_dispatch_layout(moe):
    idx, wts = random_routing(3000, 32, 4, 5, 0.1)
    x = torch.randn((3000, 64), device="cuda").to(torch.bfloat16)
    _, _, lay_d = moe.moe_dispatch(x, dev(idx), dev(wts), 32)
    _, lay_b = moe.moe_build_layout(dev(idx), dev(wts), 32)
    torch.cuda.synchronize()
    assert_layout_equal(layout_host(lay_b), layout_host(lay_d))


def test_workspace_reused_across_sizes(moe):
    """One workspace, calls in stream order with shrinking and growing shapes: the
    header each call leaves is what the next one needs."""
    shape = moe.make_shape(40000, 8, 256, 8)
    ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape, "cuda")
    for i, (n, e, k) in enumerate([(40000, 256, 8), (100, 8, 2), (40000, 256, 8), (7000, 100, 5), (0, 4, 2)]):
        idx, wts = random_routing(n, e, k, 50 + i, 0.05)
        _, lay = moe.moe_build_layout(dev(idx), dev(wts), e, workspace=ws)
        torch.cuda.synchronize()
        assert_layout_equal(layout_host(lay), oracle.layout(idx, e))


def test_unzeroed_header_is_reported_not_hung(moe):
    """A workspace whose header was not zeroed: the tickets handed out are all past
    the last tile, so every tile skips its work (nothing waits), the call reports
    counters[3] = -1 and stays inside its arrays; the following call, on the header
    that call reset, is exact again."""
    n, e, k = 5000, 64, 4
    idx, wts = random_routing(n, e, k, 77)
    shape = moe.make_shape(n, 8, e, k)
    ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape, "cuda")
    base = (ws.data_ptr() + 255) & ~255
    off = base - ws.data_ptr()
    ws[off:off + 4].copy_(torch.tensor([0x00, 0x00, 0x10, 0x00], dtype=torch.uint8))  # ticket = 1 << 20
    rows = n * k
    lay = moe.Layout.empty(n, k, e, 0, rows, "cuda")
    for t in (lay.tokens_per_expert, lay.expert_offsets, lay.ordinal, lay.assign_row, lay.row_src):
        t.fill_(0x7FFFFFFF)
    guard = torch.full((rows + 2048,), -7.0, device="cuda")
    wp = guard[1024:1024 + rows]
    _, lay = moe.moe_build_layout(dev(idx), dev(wts), e, layout=lay, w_perm_out=wp, workspace=ws)
    torch.cuda.synchronize()
    assert int(lay.counters[3].item()) == -1
    g = guard.cpu().numpy()
    assert (g[:1024] == -7.0).all() and (g[-1024:] == -7.0).all()
    assert int(ws[off:off + 4].view(torch.int32).item()) == 0          # the ticket was reset
    _, lay2 = moe.moe_build_layout(dev(idx), dev(wts), e, workspace=ws)
    torch.cuda.synchronize()
    assert_layout_equal(layout_host(lay2), oracle.layout(idx, e))
