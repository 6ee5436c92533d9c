"""moe_dispatch_noalloc (include/moe.h): the dispatch on the library's static
per-GPU scratch, for callers that cannot allocate.  Through the C ABI, its
outputs must equal moe_dispatch's bit for bit -- every layout field, the
dispatched rows, the permuted weights -- on calls in a row that reuse the
scratch with shrinking inputs (the scratch keeps the last call's state), and
on a capacity layout dropped by weight."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import assert_layout_equal, dev, host, layout_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_router_softmax_amd as m
    return m


def case(n, e, k, h, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.1] = -1
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), mi.DT_BF16, 90, seed)
    return idx, wts, x


@pytest.mark.parametrize("calls", [
    # (tokens, experts, top-k, hidden, capacity, drop policy): each call smaller than the one before
    [(6000, 256, 8, 512, 0, 0), (700, 16, 2, 256, 0, 0)],
    [(4096, 64, 4, 384, 300, 1), (1000, 64, 4, 384, 70, 1), (513, 8, 2, 128, 0, 0)],
])
def test_noalloc_dispatch_equals_dispatch(moe, calls):
    for i, (n, e, k, h, cap, pol) in enumerate(calls):
        print(f"noalloc call {i}: n={n} e={e} k={k} h={h} capacity={cap} policy={pol}", flush=True)
        idx, wts, x = case(n, e, k, h, 100 + i)
        xd, idd, wd = dev(x), dev(idx), dev(wts)
        xp_a, wp_a, lay_a = moe.moe_dispatch(xd, idd, wd, e, capacity=cap, drop_policy=pol)
        xp_b, wp_b, lay_b = moe.moe_dispatch_noalloc(xd, idd, wd, e, capacity=cap, drop_policy=pol)
        torch.cuda.synchronize()
        got, ref = layout_host(lay_b), layout_host(lay_a)
        assert_layout_equal(got, ref)
        assert_layout_equal(got, oracle.layout(idx, e, cap, 0, 0, pol, wts))
        np.testing.assert_array_equal(host(wp_b), host(wp_a))
        written = ref["row_src"] >= 0
        if cap:
            written[:] = True                     # capacity pads are zeroed rows
        xa, xb = host(xp_a), host(xp_b)
        assert (xb[written].view(np.uint8) == xa[written].view(np.uint8)).all()
        assert int(got["counters"][3]) >= 0       # the scan never gave up


def test_noalloc_dispatch_rejects_shapes_beyond_its_scratch(moe):
    import ctypes as C
    s = moe.make_shape(5_000_000, 64, 256, 8)      # 40M assignments: far more status words than 8 MiB
    p = C.c_void_p(4096)
    lay = moe.MoeLayoutC(*([4096] * 8))
    assert moe.lib.moe_dispatch_noalloc(C.byref(s), p, p, p, C.byref(lay), p, None, None) == -3
