"""Helpers for the GPU parity tests: host <-> device transfer of the seeded
inputs and the error measures the tolerances are stated in."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs as mi

# Tolerances (max relative error = max|got - ref| / max|ref| over a tensor).
TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def values(a: np.ndarray) -> np.ndarray:
    """Numeric values in float64 (bf16 bit patterns are widened exactly)."""
    if a.dtype == np.uint16:
        return mi.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    g, r = values(got), values(ref)
    denom = np.abs(r).max() if r.size else 0.0
    if denom == 0.0:
        return float(np.abs(g - r).max()) if g.size else 0.0
    return float(np.abs(g - r).max() / denom)


def tol_for(dtype_or_array) -> float:
    dt = dtype_or_array.dtype if hasattr(dtype_or_array, "dtype") else dtype_or_array
    return TOL_BF16 if dt in (np.uint16, torch.bfloat16) else TOL_F32


def layout_host(layout) -> dict:
    return {f: host(getattr(layout, f)) for f in ("tokens_per_expert", "expert_offsets", "ordinal", "assign_row",
                                                  "row_src", "drop_mask", "pad_mask", "counters")}


LAYOUT_FIELDS = ("tokens_per_expert", "expert_offsets", "ordinal", "assign_row", "row_src", "drop_mask", "pad_mask",
                 "counters")


def assert_layout_equal(got: dict, ref: dict):
    for f in LAYOUT_FIELDS:
        g, r = got[f], ref[f]
        assert g.shape == r.shape, (f, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.nonzero(g != r)[0]
            raise AssertionError(f"layout field {f} differs at {bad.size} positions, first {bad[:8]}: "
                                 f"got {g[bad[:8]]} ref {r[bad[:8]]}")


def workload_inputs(w: mi.Workload, seed: int = 0):
    """(topk_idx or None, topk_w or None, logits or None, x) as numpy arrays."""
    x = mi.activations(w, seed)
    if w.has_router:
        return None, None, mi.router_logits(w, seed), x
    idx, wts = mi.received_routing(w, seed)
    return idx, wts, None, x


def every_value_at_every_scale():
    """bf16 rows in 32-element blocks: for each exponent field f_a = 0..254 the
    blocks hold the largest value of that field (the block maximum, so the
    scale code is max(f_a - 8, 0): every code a finite block can have) and,
    both signs, every pattern of the 21 exponent fields f_a - 20 .. f_a (from
    the largest codes down through E4M3's subnormals to values that round to
    zero), the last block of each f_a filled up with zeros."""
    blocks = []
    for fa in range(255):
        top = (fa << 7) | 0x7F
        lo = max(fa - 20, 0) << 7
        mag = np.arange(lo, top + 1, dtype=np.uint32)
        vals = np.concatenate([mag, mag | 0x8000]).astype(np.uint16)
        nb = -(-vals.size // 31)
        body = np.zeros(nb * 31, np.uint16)
        body[:vals.size] = vals
        blk = np.empty((nb, 32), np.uint16)
        blk[:, 0] = top
        blk[:, 1:] = body.reshape(nb, 31)
        blocks.append(blk)
    b = np.concatenate(blocks)
    pad = -b.shape[0] % 32
    b = np.concatenate([b, np.zeros((pad, 32), np.uint16)])
    return b.reshape(-1, 32 * 32)                                   # rows of 1024 elements
