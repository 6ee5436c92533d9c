"""Robustness of the C ABI on the GPU:

* two whole layer chains (route -> dispatch -> grouped FFN -> combine ->
  combine backward -> FFN backward -> dispatch backward) in flight at once on two
  streams with their own workspaces give, bit for bit, what each gives alone --
  the library keeps no shared staging state between calls (the single shared
  staging region of the MORI dispatcher, which made two dispatches in flight
  unsafe, is the lesson);
* guard regions around every output of dispatch, MXFP8 dispatch, layout,
  combine, combine backward, dispatch backward and the FFN forward and backward
  stay untouched (the out-of-bounds write and read fixes of that pull request's
  commit log are the lesson)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # guard bytes on each side of an output
FILL = 0x5A           # guard byte pattern


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


class Guarded:
    """Device tensors carved out of byte buffers with FILL-patterned guards on both sides."""

    def __init__(self):
        self.bufs = []

    def empty(self, shape, dtype):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((nbytes + 2 * GUARD,), FILL, dtype=torch.uint8, device="cuda")
        self.bufs.append((buf, nbytes))
        return buf[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def check(self):
        for i, (buf, nbytes) in enumerate(self.bufs):
            b = buf.cpu().numpy()
            assert (b[:GUARD] == FILL).all() and (b[GUARD + nbytes:] == FILL).all(), f"guard {i} overwritten"


def layer_inputs(seed, n=600, e=16, k=4, h=256, inter=128):
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter)
    logits = dev(mi.router_logits(w, seed))
    x = dev(mi.activations(w, seed))
    wgu, wd = (dev(a) for a in mi.expert_weights(w, seed))
    go = dev(mi.grad_output(w, seed))
    return dict(logits=logits, x=x, wgu=wgu, wd=wd, go=go, k=k, e=e)


def run_layer(moe, d, capacity=0):
    """The whole layer and its backward on the current stream -> dict of outputs."""
    r = moe.moe_route(d["logits"], d["k"])
    xp, wp, lay = moe.moe_dispatch(d["x"], r.topk_idx, r.topk_w, d["e"], capacity=capacity)
    y, gu = moe.moe_expert_ffn(xp, lay, d["wgu"], d["wd"], save_gate_up=True)
    out = moe.moe_combine(y, r.topk_w, lay)
    gy, gw = moe.moe_combine_bwd(d["go"], y, r.topk_w, lay)
    gxp, dwgu, dwd = moe.moe_expert_ffn_bwd(xp, gy, lay, d["wgu"], d["wd"], gate_up=gu)
    gx = moe.moe_dispatch_bwd(gxp, lay)
    kept = lay.pad_mask == 0
    return dict(idx=r.topk_idx, w=r.topk_w, assign_row=lay.assign_row, xp=xp[kept], y=y[kept], out=out,
                gy=gy[kept], gw=gw, gxp=gxp[kept], dwgu=dwgu, dwd=dwd, gx=gx)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("capacity", [0, 150])
def test_two_layer_chains_in_flight_on_two_streams(moe, capacity):
    da, db = layer_inputs(1), layer_inputs(2, n=900, e=16, k=4)
    ref_a = run_layer(moe, da, capacity)
    ref_b = run_layer(moe, db, capacity)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    for rep in range(3):
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            outs["a"] = run_layer(moe, da, capacity)
        with torch.cuda.stream(sb):
            outs["b"] = run_layer(moe, db, capacity)
        torch.cuda.current_stream().wait_stream(sa)
        torch.cuda.current_stream().wait_stream(sb)
        torch.cuda.synchronize()
        for name, ref in (("a", ref_a), ("b", ref_b)):
            for key in ref:
                assert same_bits(outs[name][key], ref[key]), (rep, name, key)


@pytest.mark.parametrize("capacity,align", [(0, 0), (40, 0), (0, 16)])
def test_outputs_stay_inside_their_buffers(moe, capacity, align):
    n, e, k, h, inter = 700, 16, 4, 256, 128
    d = layer_inputs(3, n=n, e=e, k=k, h=h, inter=inter)
    r = moe.moe_route(d["logits"], k)
    shape = moe.make_shape(n, h, e, k, capacity, 0, 0, moe.MOE_DT_BF16, align)
    rows = int(moe.lib.moe_layout_rows(__import__("ctypes").byref(shape)))
    g = Guarded()
    i32, u8 = torch.int32, torch.uint8
    lay = moe.Layout(n, k, e, capacity, rows, g.empty((e,), i32), g.empty((e + 1,), i32), g.empty((n * k,), i32),
                     g.empty((n * k,), i32), g.empty((rows,), i32), g.empty((n * k,), u8), g.empty((rows,), u8),
                     g.empty((4,), i32), align)
    xp, wp = g.empty((rows, h), torch.bfloat16), g.empty((rows,), torch.float32)
    moe.moe_dispatch(d["x"], r.topk_idx, r.topk_w, e, capacity=capacity, row_align=align, layout=lay, x_perm=xp,
                     w_perm_out=wp)
    q8, s8 = g.empty((rows, h), u8), g.empty((rows, h // 32), u8)
    lay8 = moe.Layout.empty(n, k, e, capacity, rows, "cuda", align)
    moe.moe_dispatch_mxfp8(d["x"], r.topk_idx, r.topk_w, e, capacity=capacity, row_align=align, layout=lay8,
                           x_perm_q=q8, x_perm_scale=s8, w_perm_out=g.empty((rows,), torch.float32))
    layb = moe.Layout(n, k, e, capacity, rows, g.empty((e,), i32), g.empty((e + 1,), i32), g.empty((n * k,), i32),
                      g.empty((n * k,), i32), g.empty((rows,), i32), g.empty((n * k,), u8), g.empty((rows,), u8),
                      g.empty((4,), i32), align)
    moe.moe_build_layout(r.topk_idx, r.topk_w, e, hidden=h, capacity=capacity, row_align=align, layout=layb,
                         w_perm_out=g.empty((rows,), torch.float32))
    y, gu = g.empty((rows, h), torch.bfloat16), g.empty((rows, 2 * inter), torch.bfloat16)
    moe.moe_expert_ffn(xp, lay, d["wgu"], d["wd"], y=y, gate_up=gu)
    out = g.empty((n, h), torch.bfloat16)
    moe.moe_combine(y, r.topk_w, lay, out=out)
    gy, gw = g.empty((rows, h), torch.bfloat16), g.empty((n, k), torch.float32)
    moe.moe_combine_bwd(d["go"], y, r.topk_w, lay, grad_y=gy, grad_w=gw)
    gxp = g.empty((rows, h), torch.bfloat16)
    dwgu, dwd = g.empty(tuple(d["wgu"].shape), torch.bfloat16), g.empty(tuple(d["wd"].shape), torch.bfloat16)
    moe.moe_expert_ffn_bwd(xp, gy, lay, d["wgu"], d["wd"], gate_up=gu, grad_x_perm=gxp, grad_w_gate_up=dwgu,
                           grad_w_down=dwd)
    gx = g.empty((n, h), torch.bfloat16)
    moe.moe_dispatch_bwd(gxp, lay, out=gx)
    torch.cuda.synchronize()
    g.check()
    # and the guarded run computed the right layout
    ref = oracle.layout(r.topk_idx.cpu().numpy(), e, capacity, 0, align)
    np.testing.assert_array_equal(lay.assign_row.cpu().numpy(), ref["assign_row"])
    np.testing.assert_array_equal(layb.row_src.cpu().numpy(), ref["row_src"])
