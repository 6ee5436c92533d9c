#!/usr/bin/env python3
"""Benchmark of the single-GPU MoE path on MI355X.

Headline: dispatch + combine at 4096 tokens, hidden 7168, 256 experts, top-8,
bf16 activations, fp32 N(0,1) router logits, identity expert (the
dispatch/combine shape of the mscclpp high-throughput MoE validation).  One
step = moe_route -> moe_dispatch -> moe_combine on inputs already resident in
HBM; value = algorithmic dispatch+combine bytes per step / step time (route
time included).  Also reported: per-call times, combine backward on the same
shape, and the grouped SwiGLU expert GEMM (TFLOP/s) at the Qwen3-235B-A22B-like
layer (N=8192 H=4096 E=128 k=8 I=1536) and the DeepSeek-V3-like expert share
(32 experts, H=7168, I=2048, 32768 Zipf(1.2) rows).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk/CU)
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 MFMA (twice the bf16 rate)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def events_ms(pairs):
    return [s.elapsed_time(e) for s, e in pairs]


def median(v):
    v = sorted(v)
    return v[len(v) // 2] if v else float("nan")


def pct(v, q):
    """q-th percentile (nearest rank) of v."""
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q / 100.0 * (len(v) - 1)))))] if v else float("nan")


def queue_ahead(torch, calls):
    """A compute-only spin kernel (about 40 us of GPU clock per call to be queued)
    ahead of a timed batch: every call is queued before the start event, so the
    events time the GPU, not the host issuing calls whose kernels take less time
    than their issue (the tiny workload, the router, the layout alone).  Without
    torch's spin kernel the batch is timed as issued."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(calls * 80_000))


def bench_dispatch_combine(moe, mi, torch, steps, warmup, options=True):
    import numpy as np
    w = mi.workload(2)
    logits = torch.from_numpy(mi.router_logits(w)).cuda()
    x_np = mi.activations(w)
    x = torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16)
    n, k, e, h = w.n_tokens, w.top_k, w.n_experts, w.hidden
    dev = x.device
    r = moe.moe_route(logits, k)
    xp, wp, lay = moe.moe_dispatch(x, r.topk_idx, r.topk_w, e)
    shape = moe.make_shape(n, h, e, k, act_dtype=moe.MOE_DT_BF16)
    ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape, dev)
    out = torch.empty_like(x)
    go = torch.randn(x.shape, generator=torch.Generator(device=dev).manual_seed(4), device=dev).to(torch.bfloat16)
    gy = torch.empty_like(xp)
    gw = torch.empty((n, k), dtype=torch.float32, device=dev)

    route = lambda: moe.moe_route(logits, k, out=r)
    dispatch = lambda: moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, layout=lay, x_perm=xp, w_perm_out=wp,
                                        workspace=ws)
    combine = lambda: moe.moe_combine(xp, r.topk_w, lay, out=out)

    def step():
        route()
        dispatch()
        combine()

    # The timed steps carry no event markers between the calls: a recorded event
    # costs the stream several microseconds of idle time (measured 8.6 us for an
    # empty pair), so per-call times come from runs of back-to-back calls below.
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    def b2b_ms(fns, n):
        """Mean time of n rounds of the calls fns, back to back on the stream."""
        for _ in range(warmup):
            for f in fns: f()
        torch.cuda.synchronize()
        queue_ahead(torch, n * len(fns))
        t0.record()
        for _ in range(n):
            for f in fns: f()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    route_ms = b2b_ms([route], steps)
    disp_ms = b2b_ms([dispatch], steps)
    comb_ms = b2b_ms([combine], steps)
    # dispatch then combine, in batches (one event pair per batch) for the spread
    batch = max(1, steps // 10)
    dc_batches = [b2b_ms([dispatch, combine], batch) for _ in range(10)]
    dc_ms = median(dc_batches)
    # the same step captured once in a HIP graph and replayed (no launch overhead on the host)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    graph_ms = t0.elapsed_time(t1) / steps
    del graph
    counters = lay.counters.cpu().tolist()
    kept = counters[0]
    row_b = h * 2
    dispatch_bytes = n * row_b + kept * row_b
    combine_bytes = kept * row_b + n * row_b
    # combine backward on the same layout (y = x_perm: identity expert)
    for _ in range(warmup):
        moe.moe_combine_bwd(go, xp, r.topk_w, lay, grad_y=gy, grad_w=gw)
    torch.cuda.synchronize()
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    b0.record()
    for _ in range(steps):
        moe.moe_combine_bwd(go, xp, r.topk_w, lay, grad_y=gy, grad_w=gw)
    b1.record()
    torch.cuda.synchronize()
    bwd_ms = b0.elapsed_time(b1) / steps
    bwd_bytes = n * row_b + kept * row_b * 2
    # dispatch backward (grad of the token rows) on the same layout
    gx = torch.empty_like(x)
    for _ in range(warmup):
        moe.moe_dispatch_bwd(gy, lay, out=gx)
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(steps):
        moe.moe_dispatch_bwd(gy, lay, out=gx)
    d1.record()
    torch.cuda.synchronize()
    dbwd_ms = d0.elapsed_time(d1) / steps
    # MXFP8 dispatch (rows quantised to E4M3 + one E8M0 scale per 32 elements on the way)
    q8 = torch.empty((xp.shape[0], h), dtype=torch.uint8, device=dev)
    s8 = torch.empty((xp.shape[0], h // 32), dtype=torch.uint8, device=dev)
    lay8 = moe.Layout.empty(n, k, e, 0, xp.shape[0], dev)

    def mx_dispatch():
        moe.moe_dispatch_mxfp8(x, r.topk_idx, r.topk_w, e, layout=lay8, x_perm_q=q8, x_perm_scale=s8,
                               w_perm_out=wp, workspace=ws)

    for _ in range(warmup):
        mx_dispatch()
    torch.cuda.synchronize()
    d0.record()
    for _ in range(steps):
        mx_dispatch()
    d1.record()
    torch.cuda.synchronize()
    mx_ms = d0.elapsed_time(d1) / steps
    mx_bytes = n * row_b + kept * (h + h // 32)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    # the force-balanced router (random logits drawn on the device) at the same shape
    rr = moe.moe_route_random(n, e, k, 7, device=dev)
    for _ in range(warmup):
        moe.moe_route_random(n, e, k, 7, device=dev, out=rr)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(steps):
        moe.moe_route_random(n, e, k, 7, device=dev, out=rr)
    c1.record()
    torch.cuda.synchronize()
    route_random_ms = c0.elapsed_time(c1) / steps
    # cold caches: before each timed step, outside the timed region, read 1 GiB
    # (evicts the 4 MB L2 of every XCD and the 256 MB MALL, which could hold x;
    # a read leaves clean lines, so no write-back of the flush lands in the step)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    # cold dispatch + combine: one event pair around the two calls; the split
    # between them comes from a second pass with a marker in between
    def cold_pass(split):
        # the flush is queued without a host synchronisation, so the host has
        # enqueued the whole step before the GPU reaches it: the events time the
        # GPU, not the host's launch latency
        res = []
        for _ in range(min(steps, 20)):
            flush.sum()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            route()
            ev[1].record()
            dispatch()
            if split:
                ev[2].record()
            combine()
            ev[3].record()
            torch.cuda.synchronize()
            res.append(ev)
        return res
    cold = cold_pass(False)
    cold_route = [r_[0].elapsed_time(r_[1]) for r_ in cold]
    cold_dc = [r_[1].elapsed_time(r_[3]) for r_ in cold]
    cold = cold_pass(True)
    cold_disp = [r_[1].elapsed_time(r_[2]) for r_ in cold]
    cold_comb = [r_[2].elapsed_time(r_[3]) for r_ in cold]
    # a plain device copy of 1 GiB (2.15 GB moved) for the measured-bandwidth fraction
    dst = torch.empty_like(flush)
    dst.copy_(flush)
    torch.cuda.synchronize()
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record()
    for _ in range(5):
        dst.copy_(flush)
    k1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * flush.numel() * 4 / (k0.elapsed_time(k1) / 5 * 1e-3) / 1e9
    del flush, dst
    if not options:
        return dict(total_ms=total_ms, kept=kept)
    # router and layout options at the same shape, back to back: a selection-only
    # expert bias, a padding-token mask (every tenth token), and dropless segments
    # aligned to 128 rows (the zeroed pad rows between segments are written too)
    g = torch.Generator(device=dev).manual_seed(11)
    bias = torch.randn(e, generator=g, device=dev) * 0.1
    rb = moe.moe_route(logits, k, expert_bias=bias)
    mask = (torch.arange(n, device=dev) % 10 == 0).to(torch.uint8)
    rm = moe.moe_route(logits, k, token_mask=mask)
    route_bias_ms = b2b_ms([lambda: moe.moe_route(logits, k, expert_bias=bias, out=rb)], steps)
    route_mask_ms = b2b_ms([lambda: moe.moe_route(logits, k, token_mask=mask, out=rm)], steps)
    xpa, wpa, laya = moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, row_align=128)
    shape_a = laya.shape(h, moe.MOE_DT_BF16)
    ws_a = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape_a, dev)
    aligned_ms = b2b_ms([lambda: moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, row_align=128, layout=laya, x_perm=xpa,
                                                  w_perm_out=wpa, workspace=ws_a)], steps)
    aligned_rows = int(laya.expert_offsets[e].item())
    del xpa, wpa, laya, ws_a
    return dict(total_ms=total_ms, route_ms=route_ms, dispatch_ms=disp_ms, combine_ms=comb_ms,
                route_bias_ms=route_bias_ms, route_mask_ms=route_mask_ms, aligned_ms=aligned_ms,
                aligned_rows=aligned_rows,
                comb_kernel_ms=comb_ms, kept=kept, copy_gbs=copy_gbs, dbwd_ms=dbwd_ms,
                route_random_ms=route_random_ms, graph_ms=graph_ms,
                dc_ms=dc_ms, dc_p10=pct(dc_batches, 10), dc_p90=pct(dc_batches, 90),
                cold_route_ms=median(cold_route), cold_dispatch_ms=median(cold_disp),
                cold_combine_ms=median(cold_comb), cold_dc_ms=median(cold_dc),
                cold_dc_p10=pct(cold_dc, 10), cold_dc_p90=pct(cold_dc, 90),
                dispatch_bytes=dispatch_bytes, combine_bytes=combine_bytes, bwd_ms=bwd_ms, bwd_bytes=bwd_bytes,
                mx_ms=mx_ms, mx_bytes=mx_bytes,
                n=n, k=k, e=e, h=h)


def dispatch_combine_at(moe, mi, torch, wid, steps, warmup, flush):
    """Dispatch -> combine (identity expert: the combine reads the dispatched rows) at
    workload `wid`, warm (back-to-back pairs) and cold (each pair after a 1 GiB read,
    queued without a host synchronisation) -> dict.  The tiny fp32 workload also
    times its whole step (route -> dispatch -> combine), eagerly and as a replayed
    HIP graph: it is bound by launch latency."""
    import numpy as np
    w = mi.workload(wid)
    dev = torch.device("cuda")
    xn = mi.activations(w)
    x = torch.from_numpy(xn.view(np.int16)).cuda().view(torch.bfloat16) if xn.dtype == np.uint16 else \
        torch.from_numpy(xn).cuda()
    n, k, e, h = w.n_tokens, w.top_k, w.n_experts, w.hidden
    if w.has_router:
        logits = torch.from_numpy(mi.router_logits(w)).cuda()
        r = moe.moe_route(logits, k)
        idx, wts = r.topk_idx, r.topk_w
    else:
        idx_np, w_np = mi.received_routing(w)
        idx, wts = torch.from_numpy(idx_np).cuda(), torch.from_numpy(w_np).cuda()
    max_rows = w.rows if w.rows else 0
    xp, wp, lay = moe.moe_dispatch(x, idx, wts, e, max_rows=max_rows)
    ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, lay.shape(h, moe.MOE_DT_BF16 if x.dtype == torch.bfloat16 else
                                                             moe.MOE_DT_F32), dev)
    out = torch.empty_like(x)
    disp = lambda: moe.moe_dispatch(x, idx, wts, e, max_rows=max_rows, layout=lay, x_perm=xp, w_perm_out=wp,
                                    workspace=ws)
    comb = lambda: moe.moe_combine(xp, wts, lay, out=out)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def b2b_ms(fns, reps):
        for _ in range(warmup):
            for f in fns: f()
        torch.cuda.synchronize()
        queue_ahead(torch, reps * len(fns))
        t0.record()
        for _ in range(reps):
            for f in fns: f()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    batch = max(1, steps // 10)
    warm = sorted(b2b_ms([disp, comb], batch) for _ in range(10))
    cold = []
    for _ in range(20):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        disp()
        comb()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    cold.sort()
    kept = int(lay.counters[0].item())
    eb = x.element_size()
    res = dict(workload=w.name, warm_ms=warm[5], cold_ms=cold[10], cold_p10=cold[2], cold_p90=cold[18],
               dispatch_bytes=(n + kept) * h * eb, combine_bytes=(kept + n) * h * eb, kept=kept)
    if wid == 1:
        step = lambda: (moe.moe_route(logits, k, out=r), disp(), comb())
        res["step_ms"] = b2b_ms([step], steps)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        res["graph_step_ms"] = b2b_ms([graph.replay], steps)
        del graph
    if w.backward:   # combine backward on this layout
        go = torch.from_numpy(mi.grad_output(w).view(np.int16)).cuda().view(torch.bfloat16)
        gy = torch.empty_like(xp)
        gw = torch.empty((n, k), dtype=torch.float32, device=dev)
        cb = lambda: moe.moe_combine_bwd(go, xp, wts, lay, grad_y=gy, grad_w=gw)
        res["combine_bwd_ms"] = b2b_ms([cb], steps)
        cbc = []
        for _ in range(20):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            cb()
            b.record()
            torch.cuda.synchronize()
            cbc.append(a.elapsed_time(b))
        res["combine_bwd_cold_ms"] = sorted(cbc)[10]
        res["combine_bwd_bytes"] = (n + 2 * kept) * h * eb
    return res


def bench_layout_sizes(moe, torch, steps, warmup, sizes=(4096, 32768, 65536)):
    """moe_build_layout (the single-pass scan and the row placement, no row copy) at
    N tokens, 256 experts, top-8 over force-balanced random routing -> {N: us}."""
    dev = torch.device("cuda")
    res = {}
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for n in sizes:
        r = moe.moe_route_random(n, 256, 8, 31 + n, device=dev)
        wp, lay = moe.moe_build_layout(r.topk_idx, r.topk_w, 256)
        ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, lay.shape(8, moe.MOE_DT_BF16), dev)
        run = lambda: moe.moe_build_layout(r.topk_idx, r.topk_w, 256, layout=lay, w_perm_out=wp, workspace=ws)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        queue_ahead(torch, steps)
        t0.record()
        for _ in range(steps):
            run()
        t1.record()
        torch.cuda.synchronize()
        res[n] = t0.elapsed_time(t1) / steps * 1e3
    return res


def bench_skewed_capacity(moe, mi, torch, steps, warmup):
    """Dispatch + combine at the Zipf-skewed workload with capacity 160 (many drops and
    pads), dropping by position and by weight: -> dict of us and algorithmic bytes."""
    import numpy as np
    w = mi.workload(3)
    logits = torch.from_numpy(mi.router_logits(w)).cuda()
    x_np = mi.activations(w)
    x = torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16)
    n, k, e, h = w.n_tokens, w.top_k, w.n_experts, w.hidden
    r = moe.moe_route(logits, k)
    out = torch.empty_like(x)
    res = {}
    for name, policy in (("position", moe.MOE_DROP_POSITION), ("probs", moe.MOE_DROP_PROBS)):
        xp, wp, lay = moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, capacity=w.capacity, drop_policy=policy)
        shape = lay.shape(h, moe.MOE_DT_BF16)
        ws = moe.alloc_workspace(moe.MOE_OP_DISPATCH, shape, x.device)
        run_d = lambda: moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, capacity=w.capacity, drop_policy=policy,
                                         layout=lay, x_perm=xp, w_perm_out=wp, workspace=ws)
        for _ in range(warmup):
            run_d()
            moe.moe_combine(xp, r.topk_w, lay, out=out)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for _ in range(steps):
            run_d()
        ev[1].record()
        for _ in range(steps):
            moe.moe_combine(xp, r.topk_w, lay, out=out)
        ev[2].record()
        torch.cuda.synchronize()
        cnt = lay.counters.cpu().tolist()
        kept, pads = cnt[0], cnt[2]
        row_b = h * 2
        res[name] = dict(dispatch_us=ev[0].elapsed_time(ev[1]) / steps * 1e3,
                         combine_us=ev[1].elapsed_time(ev[2]) / steps * 1e3, kept=kept, dropped=cnt[1], pads=pads,
                         dispatch_bytes=n * row_b + (kept + pads) * row_b, combine_bytes=kept * row_b + n * row_b)
    return res


def bench_expert_gemm(moe, mi, torch, wid, iters, warmup, bwd_iters=0, replicas=0):
    import numpy as np
    w = mi.workload(wid)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(1000 + wid)
    e, h, inter = w.n_experts, w.hidden, w.inter
    wgu = (torch.randn((e, 2 * inter, h), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    wd = (torch.randn((e, h, inter), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    x = torch.randn((w.n_tokens, h), generator=g, device=dev).to(torch.bfloat16)
    if w.has_router:
        logits = torch.from_numpy(mi.router_logits(w)).cuda()
        r = moe.moe_route(logits, w.top_k)
        idx, wts = r.topk_idx, r.topk_w
    else:
        idx_np, w_np = mi.received_routing(w)
        idx, wts = torch.from_numpy(idx_np).cuda(), torch.from_numpy(w_np).cuda()
    xp, wp, lay = moe.moe_dispatch(x, idx, wts, e, max_rows=w.rows)
    y = torch.empty_like(xp)
    shape = lay.shape(h, moe.MOE_DT_BF16, inter)
    ws = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN, shape, dev)
    for _ in range(warmup):
        moe.moe_expert_ffn(xp, lay, wgu, wd, y=y, workspace=ws)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        moe.moe_expert_ffn(xp, lay, wgu, wd, y=y, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    rows = int(lay.counters[0].item())
    flops = 2.0 * rows * h * 3 * inter
    out = dict(workload=w.name, rows=rows, ms=ms, tflops=flops / ms / 1e9, flops=flops)
    # the same FFN over MXFP8 operands: rows from the MXFP8 dispatch, weights
    # quantised along K by moe_mx_quantize (timed too: a once-per-weight-update cost)
    if h % 512 == 0 and inter % 512 == 0:
        q8, s8, _, lay8 = moe.moe_dispatch_mxfp8(x, idx, wts, e, max_rows=w.rows)
        gq, gs = moe.moe_mx_quantize(wgu)
        dq, ds = moe.moe_mx_quantize(wd)
        y8 = torch.empty_like(xp)
        ws8 = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN_MXFP8, shape, dev)
        for _ in range(warmup):
            moe.moe_expert_ffn_mxfp8(q8, s8, lay8, gq, gs, dq, ds, y=y8, workspace=ws8)
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            moe.moe_expert_ffn_mxfp8(q8, s8, lay8, gq, gs, dq, ds, y=y8, workspace=ws8)
        b.record()
        torch.cuda.synchronize()
        ms8 = a.elapsed_time(b) / iters
        a.record()
        moe.moe_mx_quantize(wgu, q=gq, scale=gs)
        moe.moe_mx_quantize(wd, q=dq, scale=ds)
        b.record()
        torch.cuda.synchronize()
        out.update(mxfp8_ms=ms8, mxfp8_tflops=flops / ms8 / 1e9, mxfp8_weight_quant_ms=a.elapsed_time(b))
        del q8, s8, lay8, gq, gs, dq, ds, y8, ws8
    # the same FFN over force-balanced routing (random logits, moe_route_random): every
    # expert gets about rows/E rows -- the reference point the skew is measured against
    n_bal, k_bal = (w.n_tokens, w.top_k) if w.has_router else (rows // 2, 2)
    rb = moe.moe_route_random(n_bal, e, k_bal, 1234 + wid, device=dev, routing_map=False, counts=False)
    xb = torch.randn((n_bal, h), generator=g, device=dev).to(torch.bfloat16)
    xpb, _, layb = moe.moe_dispatch(xb, rb.topk_idx, rb.topk_w, e, w_perm=False)
    yb = torch.empty_like(xpb)
    for _ in range(warmup):
        moe.moe_expert_ffn(xpb, layb, wgu, wd, y=yb, workspace=ws)
    torch.cuda.synchronize()
    a.record()
    for _ in range(iters):
        moe.moe_expert_ffn(xpb, layb, wgu, wd, y=yb, workspace=ws)
    b.record()
    torch.cuda.synchronize()
    bal_ms = a.elapsed_time(b) / iters
    bal_rows = int(layb.counters[0].item())
    out.update(balanced_ms=bal_ms, balanced_tflops=2.0 * bal_rows * h * 3 * inter / bal_ms / 1e9, balanced_rows=bal_rows)
    del rb, xb, xpb, layb, yb

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    if replicas > 0:
        # hot-expert replication: placement from the expert counts, weight sync,
        # reroute, and the FFN over masters + replica slots
        counts = lay.tokens_per_expert
        rep = moe.moe_replica_plan(counts, replicas)
        wgu_r, wd_r = moe.moe_replica_sync(wgu, wd, rep)
        phys = moe.moe_reroute(idx, e, rep)
        xp_r, _, lay_r = moe.moe_dispatch(x, phys, wts, e + replicas, max_rows=w.rows)
        y_r = torch.empty_like(xp_r)
        rr_shape = moe.make_shape(idx.shape[0], h, e, idx.shape[1])
        ws_rr = moe.alloc_workspace(moe.MOE_OP_REROUTE, rr_shape, dev)
        plan_ms = timed(lambda: moe.moe_replica_plan(counts, replicas, out=rep), iters)
        sync_ms = timed(lambda: moe.moe_replica_sync(wgu, wd, rep, w_gate_up_replica=wgu_r, w_down_replica=wd_r), iters)
        rr_ms = timed(lambda: moe.moe_reroute(idx, e, rep, out=phys, workspace=ws_rr), iters)
        ffn_r_ms = timed(lambda: moe.moe_expert_ffn_replicas(xp_r, lay_r, wgu, wd, wgu_r, wd_r, y=y_r, workspace=ws),
                         iters)
        sync_bytes = 2 * replicas * 3 * inter * h * 2          # read and write each replica's weights
        out.update(replication=dict(n_replicas=replicas, plan_us=plan_ms * 1e3, reroute_us=rr_ms * 1e3,
                                    sync_us=sync_ms * 1e3, sync_gbs=sync_bytes / sync_ms / 1e6,
                                    ffn_us=ffn_r_ms * 1e3, ffn_tflops=flops / ffn_r_ms / 1e9,
                                    max_rows_per_expert=int(counts.max().item()),
                                    max_rows_per_copy=int(lay_r.tokens_per_expert.max().item())))
        del wgu_r, wd_r, phys, xp_r, lay_r, y_r, ws_rr
    del ws
    if bwd_iters > 0:

        # training forward: also stores the pre-activations [G | U] for the backward
        gu = torch.empty((xp.shape[0], 2 * inter), dtype=torch.bfloat16, device=dev)
        ws = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN, shape, dev)
        fms = timed(lambda: moe.moe_expert_ffn(xp, lay, wgu, wd, y=y, gate_up=gu, workspace=ws), iters)
        del ws
        # backward: dy [R, H] in, grad_x_perm [R, H], grad_w_gate_up, grad_w_down out
        dy = torch.randn(xp.shape, generator=g, device=dev).to(torch.bfloat16)
        gx, dwgu, dwd = torch.empty_like(xp), torch.empty_like(wgu), torch.empty_like(wd)
        ws = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN_BWD, shape, dev)
        bwd = lambda saved: moe.moe_expert_ffn_bwd(xp, dy, lay, wgu, wd, gate_up=saved, grad_x_perm=gx,
                                                   grad_w_gate_up=dwgu, grad_w_down=dwd, workspace=ws)
        bms = timed(lambda: bwd(gu), bwd_iters)
        rms = timed(lambda: bwd(None), bwd_iters)
        # the backward's products (dA, dx, dW_down, dW_gate_up): twice the forward's
        # flops; recomputing [G | U] adds 2*rows*H*2I
        bflops = 2.0 * rows * h * 6 * inter
        out.update(fwd_save_ms=fms, bwd_ms=bms, bwd_tflops=bflops / bms / 1e9, bwd_recompute_ms=rms,
                   bwd_recompute_tflops=(bflops + 2.0 * rows * h * 2 * inter) / rms / 1e9)
        del dy, gx, dwgu, dwd, ws, gu
    del wgu, wd, x, xp, y
    torch.cuda.empty_cache()
    return out


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when the kernel source changed since the counters were taken."""
    import hashlib
    import re
    path = ROOT / "profiles" / "row_kernels_uniform_hbm_traffic.md"
    if not path.exists():
        return None
    m = re.search(r"```json\n(.*?)\n```", path.read_text(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    src = (ROOT / rec["source"]).read_bytes()
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes"].get(kernel)


def counter_pass():
    """Short run for rocprofv3 counter passes: the uniform-workload loops with three
    timed calls each, then one 1 GiB device-to-device copy as the calibration
    kernel of known size."""
    import torch
    import moe_inputs as mi
    import combine_router_softmax_amd as moe
    torch.cuda.set_device(0)
    bench_dispatch_combine(moe, mi, torch, 3, 1, options=False)
    a = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def gemm_pass():
    """Short run for rocprofv3 counter passes over the expert GEMM: the qwen3-layer
    FFN workload, one warm-up call and two measured calls."""
    import torch
    import moe_inputs as mi
    import combine_router_softmax_amd as moe
    torch.cuda.set_device(0)
    bench_expert_gemm(moe, mi, torch, 4, 2, 1)
    torch.cuda.synchronize()


def bwd_pass():
    """Short run for rocprofv3 counter passes over the expert FFN backward: the
    qwen3-layer FFN, forward and training forward twice each, then the backward
    with saved pre-activations three times and with recomputation three times."""
    import torch
    import moe_inputs as mi
    import combine_router_softmax_amd as moe
    torch.cuda.set_device(0)
    bench_expert_gemm(moe, mi, torch, 4, 1, 1, 2)
    torch.cuda.synchronize()


def power_pass():
    """Five-second phases for reading board power and shader clock from outside
    (rocm-smi / amd-smi sampled by the caller): idle, the bf16 expert FFN, the
    vendor library's batched GEMM on the uniform version of its gate/up GEMM
    (128 x [512 x 4096] x [4096 x 3072]), the MXFP8 expert FFN, and the
    uniform-workload combine.  Prints one PHASE line per phase with its wall-clock
    start and end (seconds since the epoch) and its time per call."""
    import numpy as np
    import torch
    import moe_inputs as mi
    import combine_router_softmax_amd as moe
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    w = mi.workload(4)
    g = torch.Generator(device=dev).manual_seed(5)
    e, h, inter = w.n_experts, w.hidden, w.inter
    wgu = (torch.randn((e, 2 * inter, h), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    wd = (torch.randn((e, h, inter), generator=g, device=dev) * 0.02).to(torch.bfloat16)
    x = torch.randn((w.n_tokens, h), generator=g, device=dev).to(torch.bfloat16)
    r = moe.moe_route(torch.from_numpy(mi.router_logits(w)).cuda(), w.top_k)
    xp, _, lay = moe.moe_dispatch(x, r.topk_idx, r.topk_w, e, max_rows=w.rows)
    y = torch.empty_like(xp)
    shape = lay.shape(h, moe.MOE_DT_BF16, inter)
    ws = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN, shape, dev)
    q8, s8, _, lay8 = moe.moe_dispatch_mxfp8(x, r.topk_idx, r.topk_w, e, max_rows=w.rows)
    gq, gs = moe.moe_mx_quantize(wgu)
    dq, ds = moe.moe_mx_quantize(wd)
    ws8 = moe.alloc_workspace(moe.MOE_OP_EXPERT_FFN_MXFP8, shape, dev)
    xa = torch.randn((e, 512, h), generator=g, device=dev).to(torch.bfloat16)
    wb = wgu.transpose(1, 2).contiguous()  # contiguous right operand for torch.bmm
    yb = torch.empty((e, 512, 2 * inter), dtype=torch.bfloat16, device=dev)
    w2 = mi.workload(2)
    x2 = torch.from_numpy(mi.activations(w2).view(np.int16)).cuda().view(torch.bfloat16)
    r2 = moe.moe_route(torch.from_numpy(mi.router_logits(w2)).cuda(), w2.top_k)
    xp2, _, lay2 = moe.moe_dispatch(x2, r2.topk_idx, r2.topk_w, w2.n_experts)
    out2 = torch.empty_like(x2)
    rows = int(lay.counters[0].item())
    ffn_flops = 2.0 * rows * h * 3 * inter

    def phase(name, fn, secs, flops=None):
        torch.cuda.synchronize()
        t0 = time.time()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 0
        a.record()
        while time.time() - t0 < secs:
            for _ in range(4):
                fn()
            n += 4
            torch.cuda.synchronize()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / n * 1e3
        rate = f" {flops / us / 1e6:.0f} TFLOP/s" if flops else ""
        print(f"PHASE {name} {t0:.3f} {time.time():.3f} calls {n} {us:.1f} us/call{rate}", flush=True)
        time.sleep(2)

    torch.cuda.synchronize()
    t = time.time()
    time.sleep(2)
    print(f"PHASE idle {t:.3f} {time.time():.3f}", flush=True)
    phase("expert_ffn_bf16", lambda: moe.moe_expert_ffn(xp, lay, wgu, wd, y=y, workspace=ws), 5, ffn_flops)
    phase("vendor_bmm_gate_up", lambda: torch.bmm(xa, wb, out=yb), 5, 2.0 * e * 512 * h * 2 * inter)
    phase("expert_ffn_mxfp8", lambda: moe.moe_expert_ffn_mxfp8(q8, s8, lay8, gq, gs, dq, ds, y=y, workspace=ws8), 5,
          ffn_flops)
    phase("combine_uniform", lambda: moe.moe_combine(xp2, r2.topk_w, lay2, out=out2), 5)


def host_cpu():
    """(threads this process may run, host CPU model name)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def cpu_baseline(mi, min_seconds=8.0):
    """The oracle as it stands on the host, on full uniform-workload steps (route,
    layout, scatter, combine): one step on one thread, then steps on every thread
    the process may run until min_seconds have passed -- route, scatter and combine
    split over token ranges (tokens are independent, so no per-token arithmetic is
    reordered), the layout's counting sort whole (it is sequential).  The combine
    backward of the same shape is timed once each way beside it."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    threads, model = host_cpu()
    lib = oracle.lib()
    p = oracle._p
    w = mi.workload(2)
    n, k, e, h = w.n_tokens, w.top_k, w.n_experts, w.hidden
    logits = mi.router_logits(w)
    x = mi.activations(w)
    go = mi.grad_output(w)
    row_b = h * 2
    ranges = [(n * i // threads, n * (i + 1) // threads) for i in range(threads)]
    pool = ThreadPoolExecutor(threads)

    def par(fn):
        return list(pool.map(lambda r: fn(*r), ranges))

    def step(parallel):
        t = [time.perf_counter()]
        if parallel:
            parts = par(lambda a, b: oracle.route(logits[a:b], k)[:2])
            idx = np.concatenate([q[0] for q in parts])
            wts = np.concatenate([q[1] for q in parts])
        else:
            idx, wts, _, _ = oracle.route(logits, k)
        t.append(time.perf_counter())
        lay = oracle.layout(idx, e)
        t.append(time.perf_counter())
        rows = lay["rows"]
        xp = np.empty((rows, h), np.uint16)
        ar = lay["assign_row"]
        if parallel:   # rows of distinct tokens never overlap; no pads in a dropless layout
            par(lambda a, b: lib.oracle_scatter(b - a, k, row_b, p(x[a:b]), p(ar[a * k:b * k]), p(wts[a:b]), 0,
                                                None, 0, p(xp), None))
        else:
            oracle.scatter(x, k, lay, wts, x_perm=xp)
        t.append(time.perf_counter())
        out = np.empty((n, h), np.uint16)
        if parallel:
            par(lambda a, b: lib.oracle_combine(b - a, k, h, oracle.DT_BF16, p(xp), p(wts[a:b]), p(ar[a * k:b * k]),
                                                p(out[a:b])))
        else:
            out = oracle.combine(xp, wts, lay, n, k)
        t.append(time.perf_counter())
        return np.diff(t), lay, xp, wts

    one, lay, xp, wts = step(False)
    kept = int(lay["counters"][0])
    byts = (n + kept) * row_b * 2
    steps, tot = 0, np.zeros(4)
    start = time.perf_counter()
    while steps == 0 or time.perf_counter() - start < min_seconds:
        d, _, _, _ = step(True)
        tot += d
        steps += 1
    per = tot / steps
    # combine backward: read g and the kept rows, write grad_y, grad_w (double accumulation)
    ar = lay["assign_row"]
    gy = np.empty_like(xp)
    gw = np.empty((n, k), np.float32)
    t0 = time.perf_counter()
    lib.oracle_combine_bwd(n, k, h, oracle.DT_BF16, p(go), p(xp), p(wts), p(ar), 0, None, 0, p(gy), p(gw))
    t1 = time.perf_counter()
    par(lambda a, b: lib.oracle_combine_bwd(b - a, k, h, oracle.DT_BF16, p(go[a:b]), p(xp), p(wts[a:b]),
                                            p(ar[a * k:b * k]), 0, None, 0, p(gy), p(gw[a:b])))
    t2 = time.perf_counter()
    pool.shutdown()
    bwd_bytes = (n + 2 * kept) * row_b
    ms = lambda v: f"{1e3 * v:.0f} ms"
    return dict(value=round(byts / per.sum() / 1e9, 3), unit="GB/s", cores=threads, kind="oracle",
                cpu_model=model, nproc=os.cpu_count(),
                single_thread_gbs=round(byts / one.sum() / 1e9, 3),
                combine_bwd_gbs=round(bwd_bytes / (t2 - t1) / 1e9, 3),
                combine_bwd_single_thread_gbs=round(bwd_bytes / (t1 - t0) / 1e9, 3),
                sample=f"uniform workload (4096 tokens, hidden 7168, 256 experts, top-8, bf16), full steps of "
                       f"route + layout + scatter + combine: {steps} steps on {threads} threads "
                       f"(per step: route {ms(per[0])}, layout {ms(per[1])} on one thread, scatter {ms(per[2])}, "
                       f"combine {ms(per[3])}), and one step on one thread (route {ms(one[0])}, layout "
                       f"{ms(one[1])}, scatter {ms(one[2])}, combine {ms(one[3])}); combine backward once each "
                       f"way ({ms(t2 - t1)} on {threads} threads, {ms(t1 - t0)} on one)")


def config_entry(o):
    """The bench line's entry for one of the other workloads' dispatch -> combine."""
    byts = o["dispatch_bytes"] + o["combine_bytes"]
    gbs = lambda ms: round(byts / (ms * 1e-3) / 1e9, 1)
    d = {"dispatch_combine_us": round(o["warm_ms"] * 1e3, 2), "dispatch_combine_gbs": gbs(o["warm_ms"]),
         "frac_hbm_peak": round(byts / (o["warm_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "cold_us": round(o["cold_ms"] * 1e3, 2), "cold_p10_p90_us": [round(o["cold_p10"] * 1e3, 2),
                                                                      round(o["cold_p90"] * 1e3, 2)],
         "cold_gbs": gbs(o["cold_ms"]), "cold_frac_hbm_peak": round(byts / (o["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "bytes": byts, "kept_rows": o["kept"]}
    if "step_ms" in o:
        d["step_us"] = round(o["step_ms"] * 1e3, 2)
        d["graph_step_us"] = round(o["graph_step_ms"] * 1e3, 2)
    if "combine_bwd_ms" in o:
        b = o["combine_bwd_bytes"]
        d["combine_bwd_us"] = round(o["combine_bwd_ms"] * 1e3, 2)
        d["combine_bwd_gbs"] = round(b / (o["combine_bwd_ms"] * 1e-3) / 1e9, 1)
        d["combine_bwd_frac_hbm_peak"] = round(b / (o["combine_bwd_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        d["combine_bwd_cold_us"] = round(o["combine_bwd_cold_ms"] * 1e3, 2)
        d["combine_bwd_bytes"] = b
    return d


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--gemm-iters", type=int, default=10)
    ap.add_argument("--skip-gemm", action="store_true")
    ap.add_argument("--bwd-iters", type=int, default=5, help="expert FFN backward iterations (0: skip)")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--counter-pass", action="store_true",
                    help="short run for rocprofv3 --pmc passes (prints no JSON line)")
    ap.add_argument("--gemm-pass", action="store_true",
                    help="short expert-GEMM run for hardware-counter passes (prints nothing)")
    ap.add_argument("--bwd-pass", action="store_true",
                    help="short expert-FFN backward run for hardware-counter passes (prints nothing)")
    ap.add_argument("--power-pass", action="store_true",
                    help="five-second phases for sampling board power and clock from outside (PHASE lines)")
    args = ap.parse_args()
    if args.power_pass:
        power_pass()
        return
    if args.gemm_pass:
        gemm_pass()
        return
    if args.bwd_pass:
        bwd_pass()
        return
    if args.counter_pass:
        counter_pass()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the expert-parallel all-to-all is out "
              "of scope); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs as mi
    import combine_router_softmax_amd as moe

    torch.cuda.set_device(0)
    log("dispatch+combine: uniform workload N=4096 H=7168 E=256 k=8")
    dc = bench_dispatch_combine(moe, mi, torch, args.steps, args.warmup)
    log("dispatch+combine: Zipf-skewed workload with capacity 160, both drop policies")
    skew = bench_skewed_capacity(moe, mi, torch, 20, 3)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    other = {}
    for wid in (1, 4, 5):
        log(f"dispatch+combine: workload {mi.workload(wid).name}")
        other[wid] = dispatch_combine_at(moe, mi, torch, wid, min(args.steps, 100), 5, flush)
    del flush
    log("layout alone at 4096 / 32768 / 65536 tokens")
    layout_us = bench_layout_sizes(moe, torch, min(args.steps, 100), 5)
    gemm = []
    if not args.skip_gemm:
        for wid in (4, 5):
            log(f"expert GEMM: workload {mi.workload(wid).name}")
            gemm.append(bench_expert_gemm(moe, mi, torch, wid, args.gemm_iters, 2, args.bwd_iters,
                                          replicas=8 if wid == 5 else 0))
    cpu = None
    if not args.skip_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(mi)

    step_ms = dc["total_ms"] / args.steps
    byts = dc["dispatch_bytes"] + dc["combine_bytes"]
    comb_gbs = dc["combine_bytes"] / (dc["comb_kernel_ms"] * 1e-3) / 1e9
    traffic = recorded_traffic("combine_kernel<true, 8>")
    line = {
        "metric": "dispatch+combine µs & GB/s (4096 tok, h7168, E256, top8); expert GEMM TFLOPS",
        "value": round(byts / (step_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "uniform: N=4096 tokens, hidden=7168, E=256 experts, top-8, bf16 activations, "
                               "fp32 N(0,1) logits, identity expert, dropless",
                   "step": "moe_route -> moe_dispatch -> moe_combine", "global_batch": 4096,
                   "parallelism": "single GPU"},
        "route_us": round(dc["route_ms"] * 1e3, 2),
        "dispatch_us": round(dc["dispatch_ms"] * 1e3, 2),
        "combine_us": round(dc["combine_ms"] * 1e3, 2),
        "dispatch_combine_us": round(dc["dc_ms"] * 1e3, 2),
        "dispatch_combine_gbs": round(byts / (dc["dc_ms"] * 1e-3) / 1e9, 2),
        "dispatch_combine_frac_hbm_peak": round(byts / (dc["dc_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "dispatch_combine_p10_p90_us": [round(dc["dc_p10"] * 1e3, 2), round(dc["dc_p90"] * 1e3, 2)],
        "timing": "route/dispatch/combine_us: means of back-to-back calls of each; dispatch_combine_us: median "
                  "of 10 batches of dispatch->combine pairs, one event pair per batch",
        "cold": {"route_us": round(dc["cold_route_ms"] * 1e3, 2),
                 "dispatch_us": round(dc["cold_dispatch_ms"] * 1e3, 2),
                 "combine_us": round(dc["cold_combine_ms"] * 1e3, 2),
                 "dispatch_combine_us": round(dc["cold_dc_ms"] * 1e3, 2),
                 "dispatch_combine_p10_p90_us": [round(dc["cold_dc_p10"] * 1e3, 2),
                                                 round(dc["cold_dc_p90"] * 1e3, 2)],
                 "dispatch_combine_gbs": round(byts / (dc["cold_dc_ms"] * 1e-3) / 1e9, 2),
                 "frac_hbm_peak": round(byts / (dc["cold_dc_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "note": "median of 20 steps, each after a 1 GiB read that evicts L2 and MALL; the split "
                         "from 20 more with an event between the two calls"},
        "copy_gbs": round(dc["copy_gbs"], 1),
        "dispatch_combine_frac_of_copy": round(byts / (dc["dc_ms"] * 1e-3) / 1e9 / dc["copy_gbs"], 4),
        "graph_step_us": round(dc["graph_ms"] * 1e3, 2),
        "graph_step_gbs": round(byts / (dc["graph_ms"] * 1e-3) / 1e9, 2),
        "route_force_balanced_us": round(dc["route_random_ms"] * 1e3, 2),
        "route_expert_bias_us": round(dc["route_bias_ms"] * 1e3, 2),
        "route_token_mask_us": round(dc["route_mask_ms"] * 1e3, 2),
        "dispatch_row_align_128": {"us": round(dc["aligned_ms"] * 1e3, 2), "rows": dc["aligned_rows"],
                                   "gbs": round((dc["n"] + dc["aligned_rows"]) * dc["h"] * 2
                                                / (dc["aligned_ms"] * 1e-3) / 1e9, 1)},
        "zipf_capacity": {p: {"dispatch_us": round(v["dispatch_us"], 2), "combine_us": round(v["combine_us"], 2),
                              "dispatch_gbs": round(v["dispatch_bytes"] / v["dispatch_us"] / 1e3, 1),
                              "combine_gbs": round(v["combine_bytes"] / v["combine_us"] / 1e3, 1),
                              "kept": v["kept"], "dropped": v["dropped"], "pad_rows": v["pads"]}
                          for p, v in skew.items()},
        "dispatch_bwd_us": round(dc["dbwd_ms"] * 1e3, 2),
        "dispatch_bwd_gbs": round(dc["combine_bytes"] / (dc["dbwd_ms"] * 1e-3) / 1e9, 2),
        "dispatch_mxfp8_us": round(dc["mx_ms"] * 1e3, 2),
        "dispatch_mxfp8_gbs": round(dc["mx_bytes"] / (dc["mx_ms"] * 1e-3) / 1e9, 2),
        "combine_bwd_us": round(dc["bwd_ms"] * 1e3, 2),
        "combine_bwd_gbs": round(dc["bwd_bytes"] / (dc["bwd_ms"] * 1e-3) / 1e9, 2),
        "roofline": {"kernel": "combine_kernel<true, 8>", "bound": "hbm", "achieved": round(comb_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "launch_us": round(dc["comb_kernel_ms"] * 1e3, 2),
                     "algorithmic_bytes": dc["combine_bytes"]},
        "expert_gemm": [{"workload": g["workload"], "rows": g["rows"], "us": round(g["ms"] * 1e3, 1),
                         "tflops": round(g["tflops"], 1), "frac_bf16_peak": round(g["tflops"] / BF16_PEAK_TFLOPS, 4),
                         "force_balanced_tflops": round(g["balanced_tflops"], 1),
                         "frac_of_force_balanced": round(g["tflops"] / g["balanced_tflops"], 4),
                         **({"fwd_saving_gate_up_us": round(g["fwd_save_ms"] * 1e3, 1),
                             "bwd_us": round(g["bwd_ms"] * 1e3, 1), "bwd_tflops": round(g["bwd_tflops"], 1),
                             "bwd_frac_bf16_peak": round(g["bwd_tflops"] / BF16_PEAK_TFLOPS, 4),
                             "bwd_recompute_us": round(g["bwd_recompute_ms"] * 1e3, 1),
                             "bwd_recompute_tflops": round(g["bwd_recompute_tflops"], 1)} if "bwd_ms" in g else {}),
                         **({"mxfp8_us": round(g["mxfp8_ms"] * 1e3, 1), "mxfp8_tflops": round(g["mxfp8_tflops"], 1),
                             "mxfp8_frac_fp8_peak": round(g["mxfp8_tflops"] / FP8_PEAK_TFLOPS, 4),
                             "mxfp8_speedup_vs_bf16": round(g["ms"] / g["mxfp8_ms"], 3),
                             "mxfp8_weight_quant_us": round(g["mxfp8_weight_quant_ms"] * 1e3, 1)}
                            if "mxfp8_ms" in g else {}),
                         **({"replication": {k_: (round(v, 2) if isinstance(v, float) else v)
                                             for k_, v in g["replication"].items()}} if "replication" in g else {})}
                        for g in gemm],
        "configs": {o["workload"]: config_entry(o) for o in other.values()},
        "layout_us": {f"N{n_}_E256_k8": round(v, 2) for n_, v in layout_us.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
