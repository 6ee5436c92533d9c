"""Pins for the CPU oracle: each oracle function checked against something other than
itself -- brute force with a different algorithm on tiny inputs, closed forms,
library routines and invariants of the method.  CPU only.

Sources of the checked facts:
  * Router top-k with lowest-index tie-break, softmax then renormalisation over the
    chosen k, capacity factor, SwiGLU expert: the workload definitions (not the pages).
  * Stable per-expert ordinals: DeepSpeed ep_tp_dispatch.py,
    assignment_ordinals_by_expert (segment starts where the expert id changes, a
    running maximum of the start positions, ordinal = position - segment start).
  * Drop/pad masks and "active = not dropped and not padded": DeepSpeed
    ep_tp_dispatch.py, RoutedAssignmentPayload / partition_assignments.
  * Slot-ordered weighted combine into a zeroed output: DeepSpeed
    ep_tp_dispatch.py, restore_combined.
  * Exact dispatched copies (max |got - expected| = 0): mscclpp HT commit, Validation.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import moe_inputs as mi
import oracle

RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------- brute force

def bf_topk(row: np.ndarray, k: int):
    """Python sort over (NaN last, -value with -0 == +0, index)."""
    def key(e):
        v = float(row[e])
        if math.isnan(v):
            return (1, 0.0, e)
        return (0, -(v + 0.0), e)
    return sorted(range(row.size), key=key)[:k]


def bf_weights(row: np.ndarray, sel):
    """Softmax restricted to the chosen experts (equal to softmax-then-renormalise),
    with math.fsum, in double."""
    v = [float(row[e]) for e in sel]
    m = max(v)
    ex = [math.exp(x - m) for x in v]
    s = math.fsum(ex)
    return [x / s for x in ex]


def bf_layout(idx: np.ndarray, e: int, capacity: int, max_rows: int, row_align: int = 0, probs=None):
    """Permutation by a comparison sort on (expert, assignment); ordinals by the
    segment-start / running-max construction over the expert-sorted list; with a
    row alignment A, dropless segments are the counts rounded up to multiples of A."""
    flat = idx.reshape(-1)
    a_total = flat.size
    valid = [a for a in range(a_total) if 0 <= flat[a] < e]
    order = sorted(valid, key=lambda a: (int(flat[a]), a))
    ids = np.array([flat[a] for a in order], dtype=np.int64)
    pos = np.arange(ids.size)
    if ids.size:
        seg_start = np.zeros(ids.size, bool)
        seg_start[0] = True
        seg_start[1:] = ids[1:] != ids[:-1]
        starts = np.maximum.accumulate(np.where(seg_start, pos, 0))
        ords_sorted = pos - starts
    else:
        ords_sorted = pos
    ordinal = np.full(a_total, -1, np.int64)
    for p, a in enumerate(order):
        ordinal[a] = ords_sorted[p]
    counts = np.bincount(ids, minlength=e) if ids.size else np.zeros(e, np.int64)
    if capacity > 0:
        rows = e * capacity
        offsets = np.arange(e + 1) * capacity
        kept = np.minimum(counts, capacity)
    else:
        al = max(row_align, 1)
        rows = max_rows if max_rows > 0 else a_total + e * (al - 1)
        padded = [-(-int(c) // al) * al for c in counts]
        offsets = np.minimum(np.concatenate([[0], np.cumsum(padded, dtype=np.int64)]), rows)
        kept = np.minimum(counts, rows - offsets[:-1])
    assign_row = np.full(a_total, -1, np.int64)
    drop = np.zeros(a_total, np.uint8)
    if probs is not None and capacity > 0:
        # keep each expert's C largest weights (NaN last, ties by position), rows in position order
        wf = probs.reshape(-1)
        keepset = set()
        for ex in range(e):
            mine = [a for a in valid if flat[a] == ex]
            rank = sorted(mine, key=lambda a: (1 if math.isnan(wf[a]) else 0,
                                               0.0 if math.isnan(wf[a]) else -(float(wf[a]) + 0.0), a))
            keepset |= set(rank[:capacity])
        placed = np.zeros(e, np.int64)
        for a in valid:
            ex = flat[a]
            if a in keepset:
                assign_row[a] = offsets[ex] + placed[ex]
                placed[ex] += 1
            else:
                drop[a] = 1
    else:
        for a in valid:
            ex = flat[a]
            if ordinal[a] < kept[ex]:
                assign_row[a] = offsets[ex] + ordinal[a]
            else:
                drop[a] = 1
    row_src = np.full(rows, -1, np.int64)
    for a in valid:
        if assign_row[a] >= 0:
            row_src[assign_row[a]] = a
    invalid = int(sum(1 for v in flat if v < -1 or v >= e))
    return dict(ordinal=ordinal, assign_row=assign_row, drop_mask=drop, row_src=row_src,
                pad_mask=(row_src < 0).astype(np.uint8), tokens_per_expert=kept,
                expert_offsets=offsets, counters=np.array([kept.sum(), drop.sum(), offsets[-1] - kept.sum(),
                                                           invalid]))


def dense_combine_matrix(n, k, rows, topk_w, assign_row):
    m = np.zeros((n, rows), np.float64)
    for t in range(n):
        for j in range(k):
            r = assign_row[t * k + j]
            if r >= 0:
                m[t, r] += float(topk_w[t, j])
    return m


def f32_ulp(x):
    return np.spacing(np.abs(np.float32(x)).astype(np.float32))


def bf16_vals(b):
    return mi.bf16_bits_to_f32(b).astype(np.float64)


def bf16_from_double_ref(x: np.ndarray) -> np.ndarray:
    """Independent double -> bf16 (ties to even) for normal-range values: pick the
    nearer of the two bf16 neighbours obtained by truncation, breaking ties on the
    even mantissa."""
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)      # only used to get a bracket; corrected below
    u = f.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)
    cands = np.stack([lo - 1, lo, lo + 1]).astype(np.uint32) & 0xFFFF
    vals = (cands.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = np.abs(vals - x[None])
    best = np.argmin(d, axis=0)
    dmin = d.min(axis=0)
    tie = (d == dmin[None]).sum(axis=0) > 1
    out = cands[best, np.arange(x.size)] if x.ndim == 1 else None
    if x.ndim != 1:
        raise ValueError
    for i in np.nonzero(tie)[0]:
        opts = cands[d[:, i] == dmin[i], i]
        out[i] = [o for o in opts if o % 2 == 0][0]
    return out.astype(np.uint16)


# ------------------------------------------------------------------- formats

def test_bf16_round_closed_forms():
    assert oracle.bf16_round(1.0) == 0x3F80
    assert oracle.bf16_round(-2.0) == 0xC000
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 0x3F80           # tie -> even (down)
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82       # tie -> even (up)
    assert oracle.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie
    assert oracle.bf16_round(0.0) == 0x0000
    assert oracle.bf16_round(-0.0) == 0x8000
    assert oracle.bf16_round(float("inf")) == 0x7F80
    assert oracle.bf16_round(2.0 ** -133) == 0x0001               # smallest subnormal
    assert oracle.bf16_round(3.0e38) == 0x7F62                    # largest finite range
    assert oracle.bf16_round(3.5e38) == 0x7F80                    # overflow -> inf


def test_bf16_round_matches_independent_rounding():
    x = RNG.standard_normal(4000) * np.exp(RNG.uniform(-20, 20, 4000))
    got = np.array([oracle.bf16_round(v) for v in x], np.uint16)
    np.testing.assert_array_equal(got, bf16_from_double_ref(x))
    # fp32-representable inputs: the integer trick of the input generator agrees
    f = RNG.standard_normal(4000).astype(np.float32)
    got = np.array([oracle.bf16_round(float(v)) for v in f], np.uint16)
    np.testing.assert_array_equal(got, mi.f32_to_bf16_bits(f))


# --------------------------------------------------------------------- route

def _check_route_against_brute_force(logits, k):
    idx, w, rmap, tpe = oracle.route(logits, k)
    n, e = logits.shape
    for t in range(n):
        sel = bf_topk(logits[t], k)
        assert list(idx[t]) == sel, (t, logits[t], idx[t], sel)
        if not np.isnan(logits[t]).any():
            ref = bf_weights(logits[t], sel)
            assert np.all(np.abs(w[t].astype(np.float64) - ref) <= f32_ulp(np.float32(ref)) * 1.0001), (w[t], ref)
        mrow = np.zeros(e, np.uint8)
        mrow[sel] = 1
        np.testing.assert_array_equal(rmap[t], mrow)
    np.testing.assert_array_equal(tpe, rmap.sum(axis=0))
    return idx, w, rmap, tpe


@pytest.mark.parametrize("trial", range(40))
def test_route_brute_force_random(trial):
    g = np.random.default_rng(trial)
    e = int(g.integers(1, 17))
    k = int(g.integers(1, e + 1))
    n = int(g.integers(0, 40))
    logits = g.standard_normal((n, e)).astype(np.float32)
    _check_route_against_brute_force(logits, k)


@pytest.mark.parametrize("trial", range(40))
def test_route_brute_force_ties_signed_zero_nan(trial):
    g = np.random.default_rng(1000 + trial)
    e = int(g.integers(2, 17))
    k = int(g.integers(1, e + 1))
    n = 30
    vals = np.array([-1.0, -0.0, 0.0, 1.0, np.nan], np.float32)
    p = [0.25, 0.2, 0.2, 0.25, 0.1] if trial % 2 else [0.3, 0.2, 0.2, 0.3, 0.0]
    logits = g.choice(vals, size=(n, e), p=p).astype(np.float32)
    _check_route_against_brute_force(logits, k)


def test_route_tiny_workload_brute_force():
    w = mi.workload(1)
    _check_route_against_brute_force(mi.router_logits(w), w.top_k)


def test_route_closed_forms():
    # all-equal logits: lowest indices, weights exactly 1/k for k a power of two
    for k in (1, 2, 4, 8):
        idx, w, _, _ = oracle.route(np.full((3, 16), 0.7, np.float32), k)
        assert (idx == np.arange(k)).all()
        assert (w == np.float32(1.0 / k)).all()
    # k = 1: weight exactly 1
    logits = RNG.standard_normal((50, 9)).astype(np.float32)
    idx, w, _, _ = oracle.route(logits, 1)
    assert (w == 1.0).all() and (idx[:, 0] == logits.argmax(1)).all()
    # k = E: weights are the softmax (closed form), in order of decreasing logit
    idx, w, _, _ = oracle.route(logits, 9)
    for t in range(50):
        ex = np.exp(logits[t].astype(np.float64) - logits[t].max())
        sm = ex / ex.sum()
        np.testing.assert_allclose(w[t], sm[idx[t]], rtol=2 ** -23)
        assert (np.diff(logits[t][idx[t]]) <= 0).all()
    # one dominant logit: it takes slot 0 with weight ~1
    l2 = np.zeros((4, 12), np.float32)
    l2[:, 5] = 60.0
    idx, w, _, _ = oracle.route(l2, 3)
    assert (idx[:, 0] == 5).all() and (idx[:, 1:] == [0, 1]).all()
    assert np.allclose(w[:, 0], 1.0) and (w[:, 1:] < 1e-25).all()


@pytest.mark.parametrize("trial", range(20))
def test_route_token_mask_brute_force(trial):
    """Padding tokens route nowhere; the other tokens route exactly as the brute
    force does, and the counts are the column sums over the unmasked tokens only."""
    g = np.random.default_rng(2000 + trial)
    e = int(g.integers(1, 17))
    k = int(g.integers(1, e + 1))
    n = int(g.integers(1, 40))
    logits = g.standard_normal((n, e)).astype(np.float32)
    mask = (g.random(n) < 0.3).astype(np.uint8)
    mask[0] = 1 if trial % 3 == 0 else mask[0]
    if trial == 1:
        mask[:] = 1                                   # every token is padding
    idx, w, rmap, tpe = oracle.route(logits, k, mask)
    counts = np.zeros(e, np.int64)
    for t in range(n):
        if mask[t]:
            assert (idx[t] == -1).all() and (w[t] == 0).all() and (rmap[t] == 0).all()
            continue
        sel = bf_topk(logits[t], k)
        assert list(idx[t]) == sel
        ref = bf_weights(logits[t], sel)
        assert np.all(np.abs(w[t].astype(np.float64) - ref) <= f32_ulp(np.float32(ref)) * 1.0001)
        counts[sel] += 1
        mrow = np.zeros(e, np.uint8)
        mrow[sel] = 1
        np.testing.assert_array_equal(rmap[t], mrow)
    np.testing.assert_array_equal(tpe, counts)
    # the masked routing dispatches no padding token: its rows stay out of the layout
    lay = oracle.layout(idx, e)
    assert lay["counters"][0] == (1 - mask).sum() * k and lay["counters"][3] == 0
    placed = lay["assign_row"].reshape(n, k)
    assert (placed[mask == 1] == -1).all() and (placed[mask == 0] >= 0).all()


@pytest.mark.parametrize("trial", range(20))
def test_route_expert_bias_brute_force(trial):
    """Selection by logit + bias (an fp32 sum), weights from the logits of the chosen experts."""
    g = np.random.default_rng(4000 + trial)
    e = int(g.integers(1, 17))
    k = int(g.integers(1, e + 1))
    n = int(g.integers(1, 40))
    logits = g.standard_normal((n, e)).astype(np.float32)
    bias = (g.standard_normal(e) * 0.7).astype(np.float32)
    if trial % 4 == 0:
        bias[:] = np.round(bias)                      # many ties between biased scores
        logits[:] = np.round(logits * 2) / 2
    idx, w, rmap, tpe = oracle.route(logits, k, expert_bias=bias)
    for t in range(n):
        sel = bf_topk((logits[t] + bias).astype(np.float32), k)
        assert list(idx[t]) == sel
        ref = bf_weights(logits[t], sel)
        assert np.all(np.abs(w[t].astype(np.float64) - ref) <= f32_ulp(np.float32(ref)) * 1.0001)
    np.testing.assert_array_equal(tpe, rmap.sum(0))


def test_route_expert_bias_closed_forms():
    g = np.random.default_rng(5)
    logits = g.standard_normal((64, 12)).astype(np.float32)
    ref = oracle.route(logits, 3)
    zero = oracle.route(logits, 3, expert_bias=np.zeros(12, np.float32))
    for a, b in zip(ref, zero):                        # a zero bias changes nothing
        np.testing.assert_array_equal(a, b)
    big = np.zeros(12, np.float32)
    big[7] = 100.0                                     # expert 7 is selected by every token, in slot 0
    idx, w, _, tpe = oracle.route(logits, 3, expert_bias=big)
    assert (idx[:, 0] == 7).all() and tpe[7] == 64
    for t in range(64):                                # its weight still comes from its logit
        np.testing.assert_allclose(w[t], bf_weights(logits[t], list(idx[t])), rtol=2 ** -22)


def test_philox_known_answers():
    """Philox4x32-10 known-answer vectors published with the Random123 library."""
    cases = [((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
             ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
             ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
              (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1))]
    for ctr, key, out in cases:
        assert oracle.philox4x32_10(ctr, key).tolist() == list(out)


def test_random_logits_definition_and_balance():
    n, e, seed = 4096, 256, 0x0123456789ABCDEF
    lg = oracle.random_logits(n, e, seed)
    assert lg.dtype == np.float32 and (lg >= 0).all() and (lg < 1).all()
    # spot values from the definition: word x % 4 of Philox((x/4, t, 0, 0), seed), top 24 bits
    for t, x in ((0, 0), (1, 5), (4095, 255), (77, 130)):
        w = oracle.philox4x32_10((x // 4, t, 0, 0), (seed & 0xffffffff, seed >> 32))[x % 4]
        assert lg[t, x] == np.float32((int(w) >> 8) / 16777216.0)
    # uniform logits balance the experts: counts near N*k/E = 128, weights near 1/k
    idx, w, _, tpe = oracle.route_random(n, e, 8, seed)
    assert tpe.sum() == n * 8 and abs(tpe.mean() - 128) < 1e-9
    assert tpe.min() > 128 - 6 * np.sqrt(128) and tpe.max() < 128 + 6 * np.sqrt(128)
    assert np.abs(w - 0.125).max() < 0.05
    # another seed, other logits
    assert (oracle.random_logits(8, e, seed + 1) != lg[:8]).mean() > 0.99


def test_route_invariants_uniform_workload():
    w = mi.workload(2)
    logits = mi.router_logits(w)
    idx, wt, rmap, tpe = oracle.route(logits, w.top_k)
    assert tpe.sum() == w.n_tokens * w.top_k
    np.testing.assert_array_equal(tpe, rmap.sum(0))
    assert all(len(set(r)) == w.top_k for r in idx[:512])
    s = wt.astype(np.float64).sum(1)
    assert np.abs(s - 1).max() <= 4 * 2 ** -24 * w.top_k
    # shift invariance: adding a constant keeps the choice, weights within 1e-6
    idx2, wt2, _, _ = oracle.route((logits[:256] + np.float32(3.0)).astype(np.float32), w.top_k)
    same = (idx2 == idx[:256]).all(1)
    assert same.mean() > 0.99  # adding 3.0 can merge two nearby logits into a tie after rounding
    assert np.abs(wt2[same] - wt[:256][same]).max() < 1e-6
    # slot order: logits non-increasing along the slots
    chosen = np.take_along_axis(logits, idx, 1)
    assert (np.diff(chosen, axis=1) <= 0).all()


# -------------------------------------------------------------------- layout

def _check_layout(idx, e, capacity=0, max_rows=0, row_align=0):
    got = oracle.layout(idx, e, capacity, max_rows, row_align)
    ref = bf_layout(idx, e, capacity, max_rows, row_align)
    for f in ("ordinal", "assign_row", "drop_mask", "row_src", "pad_mask", "tokens_per_expert",
              "expert_offsets", "counters"):
        np.testing.assert_array_equal(got[f], ref[f], err_msg=f)
    return got


@pytest.mark.parametrize("trial", range(60))
def test_layout_brute_force_random(trial):
    g = np.random.default_rng(2000 + trial)
    e = int(g.integers(1, 17))
    k = int(g.integers(1, 5))
    n = int(g.integers(0, 65))
    mode = trial % 4
    idx = g.integers(-1, e, size=(n, k)).astype(np.int32)
    if mode == 3 and idx.size:   # invalid ids as well
        bad = g.random(idx.shape) < 0.1
        idx[bad] = g.choice([-7, e, e + 3], size=bad.sum())
    capacity = int(g.integers(1, 6)) if mode == 1 else 0
    max_rows = int(g.integers(0, n * k + 1)) if mode == 2 else 0
    _check_layout(idx, e, capacity, max_rows)


@pytest.mark.parametrize("trial", range(30))
def test_layout_row_align_brute_force_random(trial):
    """Alignment-padded dropless segments, with and without a row budget."""
    g = np.random.default_rng(3000 + trial)
    e = int(g.integers(1, 17))
    k = int(g.integers(1, 5))
    n = int(g.integers(0, 65))
    al = int(g.choice([2, 4, 16, 64]))
    idx = g.integers(-1, e, size=(n, k)).astype(np.int32)
    max_rows = int(g.integers(0, n * k + e * al + 1)) if trial % 2 else 0
    got = _check_layout(idx, e, 0, max_rows, al)
    off, kept = got["expert_offsets"], got["tokens_per_expert"]
    rows = got["rows"]
    for x in range(e):
        if off[x] < rows:
            assert off[x] % al == 0                                   # aligned starts
        end = min(off[x] + -(-int(kept[x]) // al) * al, rows)
        assert (got["pad_mask"][off[x] + kept[x]:end] == 1).all()    # alignment pads
    if not max_rows:
        assert rows == n * k + e * (al - 1) and got["counters"][1] == 0
        assert got["counters"][2] == sum(-(-int(c) // al) * al - int(c) for c in kept)


def test_layout_row_align_closed_forms():
    # counts 5, 0, 3 with alignment 4: segments [0, 8), [8, 8), [8, 12)
    idx = np.array([[0], [0], [2], [0], [2], [0], [0], [2]], np.int32)
    got = _check_layout(idx, 3, row_align=4)
    assert got["expert_offsets"].tolist() == [0, 8, 8, 12]
    assert got["tokens_per_expert"].tolist() == [5, 0, 3]
    assert got["counters"].tolist() == [8, 0, 4, 0]
    assert got["pad_mask"][:12].tolist() == [0] * 5 + [1] * 3 + [0] * 3 + [1]
    # alignment 1 is no alignment
    for al in (0, 1):
        np.testing.assert_array_equal(oracle.layout(idx, 3, row_align=al)["assign_row"],
                                      oracle.layout(idx, 3)["assign_row"])


@pytest.mark.parametrize("trial", range(30))
def test_layout_probs_drop_policy_brute_force(trial):
    """Capacity with the probability drop policy: each expert keeps its C largest weights."""
    g = np.random.default_rng(6000 + trial)
    e = int(g.integers(1, 9))
    k = int(g.integers(1, min(e, 4) + 1))
    n = int(g.integers(0, 65))
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32).reshape(n, k)
    if n:
        idx[g.random(idx.shape) < 0.1] = -1
    w = g.random((n, k)).astype(np.float32)
    if trial % 3 == 0 and n:
        w = np.round(w * 4).astype(np.float32) / 4       # many equal weights: position breaks the ties
    if trial % 5 == 0 and n:
        w[g.random(w.shape) < 0.1] = np.nan
    cap = int(g.integers(1, 6))
    got = oracle.layout(idx, e, cap, drop_policy=1, topk_w=w)
    ref = bf_layout(idx, e, cap, 0, probs=w)
    for f in ("ordinal", "assign_row", "drop_mask", "row_src", "pad_mask", "tokens_per_expert",
              "expert_offsets", "counters"):
        np.testing.assert_array_equal(got[f], ref[f], err_msg=f)
    # the same counts, offsets and pads as the position policy; only which assignments are kept differs
    pos = oracle.layout(idx, e, cap)
    for f in ("tokens_per_expert", "expert_offsets", "counters", "pad_mask", "ordinal"):
        np.testing.assert_array_equal(got[f], pos[f], err_msg=f)


def test_layout_probs_drop_policy_skewed_workload_invariants():
    """Zipf-skewed routing with capacity 160: every over-full expert's kept weights are
    all at least its dropped ones, and the kept rows stay in assignment order."""
    w = mi.workload(3)
    idx, wts, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    got = oracle.layout(idx, w.n_experts, w.capacity, drop_policy=1, topk_w=wts)
    flat, wf = idx.reshape(-1), wts.reshape(-1)
    kept = got["assign_row"] >= 0
    for ex in range(w.n_experts):
        mine = flat == ex
        if mine.sum() <= w.capacity:
            assert kept[mine].all()
            continue
        assert kept[mine].sum() == w.capacity
        assert wf[mine & kept].min() >= wf[mine & ~kept].max()
        seg = got["row_src"][ex * w.capacity:(ex + 1) * w.capacity]
        assert (np.diff(seg) > 0).all()


def test_layout_probs_drop_policy_closed_form():
    # one expert, capacity 2, weights 0.1 0.9 0.5 0.9: keeps assignments 1 and 3 (ties by position)
    idx = np.zeros((4, 1), np.int32)
    w = np.array([[0.1], [0.9], [0.5], [0.9]], np.float32)
    got = oracle.layout(idx, 1, 2, drop_policy=1, topk_w=w)
    assert got["assign_row"].tolist() == [-1, 0, -1, 1] and got["drop_mask"].tolist() == [1, 0, 1, 0]
    assert got["row_src"].tolist() == [1, 3] and got["ordinal"].tolist() == [0, 1, 2, 3]
    # under capacity every assignment is kept, as with the position policy
    got = oracle.layout(idx, 1, 4, drop_policy=1, topk_w=w)
    assert got["assign_row"].tolist() == [0, 1, 2, 3]


def test_layout_all_to_one_expert_and_capacity_one():
    idx = np.zeros((20, 1), np.int32)
    got = _check_layout(idx, 4, capacity=1)
    assert got["counters"].tolist() == [1, 19, 3, 0]
    got = _check_layout(np.full((5, 3), 2, np.int32), 3)
    assert got["tokens_per_expert"].tolist() == [0, 0, 15]
    _check_layout(np.zeros((0, 4), np.int32), 5)
    _check_layout(np.full((6, 2), -1, np.int32), 5)


def _layout_invariants(idx, e, got, capacity):
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < e)
    sentinels = int((flat == -1).sum())
    drops = int(got["drop_mask"].sum())
    assert got["counters"][0] == idx.size - drops - sentinels - got["counters"][3]
    assert got["tokens_per_expert"].sum() == got["counters"][0]
    for x in range(e):
        o0, kx = got["expert_offsets"][x], got["tokens_per_expert"][x]
        seg = got["row_src"][o0:o0 + kx]
        assert (seg >= 0).all() and (np.diff(seg) > 0).all()          # stable: source order kept
        assert (got["ordinal"][seg] == np.arange(kx)).all()            # ordinals 0..kept-1
        if capacity:
            assert (got["row_src"][o0 + kx:o0 + capacity] == -1).all()  # pads
    kept = got["assign_row"] >= 0
    assert (got["row_src"][got["assign_row"][kept]] == np.nonzero(kept)[0]).all()  # inverse maps
    if capacity:
        assert ((got["ordinal"] >= capacity) == (got["drop_mask"] == 1)).all()
        assert got["counters"][2] == (e * capacity - got["counters"][0])
    assert (got["ordinal"][~valid] == -1).all()


@pytest.mark.parametrize("wid", [1, 2, 3, 5])
def test_layout_invariants_workloads(wid):
    w = mi.workload(wid)
    if w.has_router:
        idx, _, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    else:
        idx, _ = mi.received_routing(w)
    got = oracle.layout(idx, w.n_experts, w.capacity, w.rows)
    _layout_invariants(idx, w.n_experts, got, w.capacity)
    if wid == 5:
        assert got["counters"].tolist() == [32768, 0, 0, 0]
        assert got["tokens_per_expert"].tolist() == mi.zipf_targets(32, 32768, 1.2, 16384).tolist()
    if wid == 3:
        assert got["counters"][1] > 10000 and got["counters"][2] > 10000  # skew drops and pads


def test_layout_matches_brute_force_on_uniform_workload_sample():
    w = mi.workload(2)
    idx, _, _, _ = oracle.route(mi.router_logits(w)[:300], w.top_k)
    _check_layout(idx, w.n_experts)
    _check_layout(idx, w.n_experts, capacity=7)


# ------------------------------------------------------------------- scatter

@pytest.mark.parametrize("dt,capacity", [(mi.DT_F32, 0), (mi.DT_BF16, 0), (mi.DT_BF16, 3), (mi.DT_F32, 2)])
def test_scatter_bitwise(dt, capacity, row_align=0):
    g = np.random.default_rng(7)
    n, k, e, h = 37, 3, 6, 24
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.15] = -1
    wts = g.random((n, k)).astype(np.float32)
    x = mi.normal_activations((n, h), dt, 99, 1)
    lay = oracle.layout(idx, e, capacity, row_align=row_align)
    fill = np.full((lay["rows"], h), 7, x.dtype)    # rows the scatter does not write keep this
    xp, wp = oracle.scatter(x, k, lay, wts, x_perm=fill.copy())
    kept = np.nonzero(lay["assign_row"] >= 0)[0]
    assert (xp[lay["assign_row"][kept]].view(np.uint8) == x[kept // k].view(np.uint8)).all()
    assert (wp[lay["assign_row"][kept]] == wts.reshape(-1)[kept]).all()
    pads = lay["row_src"] < 0
    assert (wp[pads] == 0).all()
    used = np.arange(lay["rows"]) < lay["expert_offsets"][-1]
    assert (xp[pads & used].view(np.uint8) == 0).all()          # capacity or alignment pads: zero
    assert (xp[pads & ~used] == fill[pads & ~used]).all()        # the unused dropless tail: untouched
    if capacity:
        assert used.all()
    if row_align > 1:
        assert (pads & used).sum() == lay["counters"][2] > 0


def test_scatter_bitwise_row_align():
    test_scatter_bitwise(mi.DT_BF16, 0, row_align=8)


# ------------------------------------------------------ dispatch backward

def _dispatch_case(dt, capacity, seed, n=41, k=3, e=6, h=24):
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.15] = -1
    lay = oracle.layout(idx, e, capacity)
    return g, idx, lay, n, k, h


@pytest.mark.parametrize("capacity", [0, 3])
def test_dispatch_bwd_is_adjoint_of_scatter_exactly(capacity):
    # small integers: every fp32 sum below is exact, so <dx, x> = <dxp, scatter(x)> holds exactly
    g, idx, lay, n, k, h = _dispatch_case(mi.DT_F32, capacity, 31)
    x = g.integers(-8, 9, (n, h)).astype(np.float32)
    dxp = g.integers(-8, 9, (lay["rows"], h)).astype(np.float32)
    xp, _ = oracle.scatter(x, k, lay, np.ones((n, k), np.float32))
    dx = oracle.dispatch_bwd(dxp, lay, n, k)
    assert (dx.astype(np.float64) * x).sum() == (dxp.astype(np.float64) * xp).sum()


@pytest.mark.parametrize("dt,capacity", [(mi.DT_F32, 0), (mi.DT_BF16, 0), (mi.DT_BF16, 2)])
def test_dispatch_bwd_dense_matrix(dt, capacity):
    # brute force: grad_x = M @ grad_x_perm with M[t, r] = number of kept slots of t in row r
    g, idx, lay, n, k, h = _dispatch_case(dt, capacity, 32 + capacity)
    dxp = mi.normal_activations((lay["rows"], h), dt, 5, 5)
    dx = oracle.dispatch_bwd(dxp, lay, n, k)
    M = np.zeros((n, lay["rows"]))
    for a, r in enumerate(lay["assign_row"]):
        if r >= 0:
            M[a // k, r] += 1.0
    val = (lambda a: a.astype(np.float64)) if dt == mi.DT_F32 else bf16_vals
    ref = M @ val(dxp)
    got = val(dx)
    tol = (2.0 ** -22 if dt == mi.DT_F32 else 2.0 ** -7) * (M @ np.abs(val(dxp))) + 1e-30
    assert (np.abs(got - ref) <= tol).all()
    none_kept = (lay["assign_row"].reshape(n, k) < 0).all(1)
    assert (dx[none_kept].view(np.uint8) == 0).all()


def test_dispatch_bwd_single_slot_is_inverse_permutation():
    g, idx, lay, n, k, h = _dispatch_case(mi.DT_BF16, 0, 33, k=1)
    dxp = mi.normal_activations((lay["rows"], h), mi.DT_BF16, 6, 6)
    dx = oracle.dispatch_bwd(dxp, lay, n, 1)
    kept = lay["assign_row"] >= 0
    assert (dx[kept].view(np.uint8) == dxp[lay["assign_row"][kept]].view(np.uint8)).all()


# ------------------------------------------------------------------- combine

@pytest.mark.parametrize("dt", [mi.DT_F32, mi.DT_BF16])
@pytest.mark.parametrize("capacity", [0, 2])
def test_combine_dense_matrix(dt, capacity):
    g = np.random.default_rng(11 + capacity)
    n, k, e, h = 29, 4, 7, 40
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[g.random(idx.shape) < 0.1] = -1
    wts = g.random((n, k)).astype(np.float32)
    lay = oracle.layout(idx, e, capacity)
    y = mi.normal_activations((lay["rows"], h), dt, 5, 5)
    out = oracle.combine(y, wts, lay, n, k)
    yv = y.astype(np.float64) if dt == mi.DT_F32 else bf16_vals(y)
    ref = dense_combine_matrix(n, k, lay["rows"], wts, lay["assign_row"]) @ yv
    if dt == mi.DT_F32:
        bound = k * 2.0 ** -24 * (np.abs(dense_combine_matrix(n, k, lay["rows"], wts, lay["assign_row"])) @ np.abs(yv)) + 1e-30
        assert (np.abs(out.astype(np.float64) - ref) <= bound).all()
    else:
        got = bf16_vals(out)
        # one bf16 rounding of an fp32 sum within k fp32 ulps of the exact value
        assert (np.abs(got - ref) <= np.abs(ref) * (2.0 ** -8 + k * 2.0 ** -23) + 1e-30).all()
    # a token with no kept slot gets a zero row
    none = np.all(lay["assign_row"].reshape(n, k) < 0, axis=1)
    if none.any():
        assert (out[none].view(np.uint8) == 0).all()


def test_combine_identity_expert_returns_input():
    # combine(dispatch(x)) == x for an identity expert and renormalised weights:
    # bitwise for bf16 (the fp32 sum lies within a few fp32 ulps of x, far inside
    # half a bf16 ulp), within k fp32 ulps for fp32.
    for wid in (1, 2):
        w = mi.workload(wid, n_tokens=256 if wid == 2 else 64, hidden=256 if wid == 2 else 128)
        logits = mi.router_logits(w)
        idx, wts, _, _ = oracle.route(logits, w.top_k)
        x = mi.activations(w)
        lay = oracle.layout(idx, w.n_experts)
        xp, _ = oracle.scatter(x, w.top_k, lay, wts)
        out = oracle.combine(xp, wts, lay, w.n_tokens, w.top_k)
        if w.dtype == mi.DT_BF16:
            assert (out == x).all()
        else:
            assert np.abs(out - x).max() <= (w.top_k + 1) * 2.0 ** -23 * np.abs(x).max()


def test_combine_exact_half_half():
    x = mi.normal_activations((10, 16), mi.DT_BF16, 3, 3)
    idx = np.array([[0, 1]] * 10, np.int32)
    lay = oracle.layout(idx, 2)
    xp, _ = oracle.scatter(x, 2, lay, np.full((10, 2), 0.5, np.float32))
    out = oracle.combine(xp, np.full((10, 2), 0.5, np.float32), lay, 10, 2)
    assert (out == x).all()


def test_combine_capacity_reduces_to_kept_weights():
    w = mi.workload(3, n_tokens=512, hidden=64)
    idx, wts, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    lay = oracle.layout(idx, w.n_experts, w.capacity)
    x = mi.normal_activations((w.n_tokens, w.hidden), mi.DT_F32, 3, 1)
    xp, _ = oracle.scatter(x, w.top_k, lay, wts)
    out = oracle.combine(xp, wts, lay, w.n_tokens, w.top_k)
    kept_w = np.where(lay["assign_row"].reshape(w.n_tokens, w.top_k) >= 0, wts, 0).astype(np.float64).sum(1)
    np.testing.assert_allclose(out, x * kept_w[:, None], rtol=1e-5, atol=1e-6)


# ------------------------------------------------------------ combine backward

@pytest.mark.parametrize("dt", [mi.DT_F32, mi.DT_BF16])
def test_combine_bwd_adjoint_euler_and_finite_differences(dt):
    g = np.random.default_rng(21)
    n, k, e, h, cap = 23, 3, 5, 32, 4
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    wts = g.random((n, k)).astype(np.float32)
    lay = oracle.layout(idx, e, cap)
    y = mi.normal_activations((lay["rows"], h), dt, 8, 8)
    go = mi.normal_activations((n, h), dt, 9, 9)
    gy, gw = oracle.combine_bwd(go, y, wts, lay, k)
    val = (lambda a: a.astype(np.float64)) if dt == mi.DT_F32 else bf16_vals
    yv, gv, gyv = val(y), val(go), val(gy)
    M = dense_combine_matrix(n, k, lay["rows"], wts, lay["assign_row"])
    out64 = M @ yv
    # adjoint: <combine(y), g> = <y, grad_y>   (combine is linear in y)
    lhs = (out64 * gv).sum()
    rhs = (yv * gyv).sum()
    rel = 2.0 ** -23 if dt == mi.DT_F32 else 2.0 ** -8
    assert abs(lhs - rhs) <= rel * (np.abs(yv) * np.abs(gyv)).sum() + 1e-12
    # Euler: sum_tj w * grad_w = <out, g>   (combine is linear in w)
    euler = (wts.astype(np.float64) * gw.astype(np.float64)).sum()
    assert abs(euler - lhs) <= 1e-6 * (np.abs(out64) * np.abs(gv)).sum()
    # central finite differences of L(w) = <combine(y, w), g> in fp64
    for t in range(n):
        for j in range(k):
            eps = 1e-3
            wp, wm = wts.astype(np.float64).copy(), wts.astype(np.float64).copy()
            wp[t, j] += eps
            wm[t, j] -= eps
            fd = (((dense_combine_matrix(n, k, lay["rows"], wp, lay["assign_row"]) @ yv) * gv).sum()
                  - ((dense_combine_matrix(n, k, lay["rows"], wm, lay["assign_row"]) @ yv) * gv).sum()) / (2 * eps)
            assert abs(fd - gw[t, j]) <= 1e-6 * (1 + abs(fd)), (t, j, fd, gw[t, j])
    # pads of grad_y are zero; dropped slots have zero grad_w
    assert (gy[lay["row_src"] < 0].view(np.uint8) == 0).all()
    assert (gw.reshape(-1)[lay["assign_row"] < 0] == 0).all()


def test_combine_bwd_identity_expert():
    w = mi.workload(2, n_tokens=64, hidden=96)
    idx, wts, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    lay = oracle.layout(idx, w.n_experts)
    x = mi.activations(w)
    xp, _ = oracle.scatter(x, w.top_k, lay, wts)
    go = mi.grad_output(w)
    gy, gw = oracle.combine_bwd(go, xp, wts, lay, w.top_k)
    ref = (bf16_vals(go) * bf16_vals(x)).sum(1)
    np.testing.assert_allclose(gw, np.repeat(ref[:, None], w.top_k, 1), rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- expert FFN

def ffn_numpy(xv, wg, wu, wd):
    """fp64 numpy matmuls with bf16 rounding of the intermediate and output."""
    gg = xv @ wg.T
    uu = xv @ wu.T
    act = bf16_vals(bf16_from_double_ref((gg / (1 + np.exp(-gg)) * uu).reshape(-1))).reshape(gg.shape)
    return bf16_from_double_ref((act @ wd.T).reshape(-1)).reshape(xv.shape[0], wd.shape[0])


def _small_ffn_case(e=3, n=40, k=2, h=48, inter=32, seed=0, same_weights=False):
    w = mi.workload(4, n_tokens=n, hidden=h, n_experts=e, top_k=k, inter=inter)
    idx, wts, _, _ = oracle.route(mi.router_logits(w, seed), k)
    lay = oracle.layout(idx, e)
    x = mi.normal_activations((n, h), mi.DT_BF16, 4, 1, seed)
    xp, _ = oracle.scatter(x, k, lay, wts)
    wgu, wd = mi.expert_weights(w, seed)
    wgu = wgu.copy()
    wd = wd.copy()
    if same_weights:
        wgu[:] = wgu[0]
        wd[:] = wd[0]
    return w, idx, wts, lay, x, xp, wgu, wd


def test_ffn_matches_numpy_matmul_per_expert():
    w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case()
    y = oracle.expert_ffn(xp, lay, wgu, wd)
    inter = w.inter
    for e in range(w.n_experts):
        o0, kx = lay["expert_offsets"][e], lay["tokens_per_expert"][e]
        if kx == 0:
            continue
        ref = ffn_numpy(bf16_vals(xp[o0:o0 + kx]), bf16_vals(wgu[e, :inter]), bf16_vals(wgu[e, inter:]),
                        bf16_vals(wd[e]))
        got = y[o0:o0 + kx]
        assert (got == ref).mean() > 0.97
        assert np.abs(bf16_vals(got) - bf16_vals(ref)).max() <= 2e-2 * np.abs(bf16_vals(ref)).max()


def test_ffn_segments_match_the_row_loop():
    """The segment-wise fp64 FFN (library matmuls) against the C row loop and the
    numpy form above: the same two roundings, sums in another order, so equal bits
    but for rare rounding boundaries, and never more than one bf16 step apart."""
    for seed, e, n, h, inter in ((0, 3, 40, 48, 32), (1, 5, 300, 128, 96), (2, 1, 70, 64, 64)):
        w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case(e=e, n=n, k=min(2, e), h=h, inter=inter, seed=seed)
        ref = oracle.expert_ffn(xp, lay, wgu, wd)
        seen = 0
        for ex, o, y in oracle.expert_ffn_segments(xp, lay, wgu, wd):
            c = int(lay["tokens_per_expert"][ex])
            assert o == lay["expert_offsets"][ex] and y.shape == (c, h)
            got, want = y, ref[o:o + c]
            assert (got == want).mean() > 0.97
            assert np.abs(bf16_vals(got) - bf16_vals(want)).max() <= 2.0 ** -7 * np.abs(bf16_vals(want)).max()
            np_ref = ffn_numpy(bf16_vals(xp[o:o + c]), bf16_vals(wgu[ex, :inter]), bf16_vals(wgu[ex, inter:]),
                               bf16_vals(wd[ex]))
            assert (got == np_ref).mean() > 0.97
            seen += c
        assert seen == int(lay["tokens_per_expert"].sum())
    only = list(oracle.expert_ffn_segments(xp, lay, wgu, wd, experts=[0]))
    assert [v[0] for v in only] == ([0] if lay["tokens_per_expert"][0] else [])


def test_ffn_single_expert_is_plain_gemm_pair():
    w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case(e=1, k=1, n=30)
    y = oracle.expert_ffn(xp, lay, wgu, wd)
    ref = ffn_numpy(bf16_vals(x), bf16_vals(wgu[0, :w.inter]), bf16_vals(wgu[0, w.inter:]), bf16_vals(wd[0]))
    assert (y == ref).mean() > 0.97


def test_ffn_zero_gate_or_up_gives_zero():
    w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case()
    z = wgu.copy()
    z[:, :w.inter] = 0
    assert (oracle.expert_ffn(xp, lay, z, wd) == 0).all()
    z = wgu.copy()
    z[:, w.inter:] = 0
    y = oracle.expert_ffn(xp, lay, z, wd)
    assert (bf16_vals(y) == 0).all()


def test_ffn_identical_experts_commute_with_permutation():
    w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case(same_weights=True)
    y = oracle.expert_ffn(xp, lay, wgu, wd)
    dense = oracle.expert_ffn(x, dict(expert_offsets=np.array([0] + [w.n_tokens] * w.n_experts, np.int32),
                                      tokens_per_expert=np.array([w.n_tokens] + [0] * (w.n_experts - 1), np.int32),
                                      pad_mask=np.zeros(w.n_tokens, np.uint8), rows=w.n_tokens), wgu, wd)
    kept = lay["assign_row"] >= 0
    np.testing.assert_array_equal(y[lay["assign_row"][kept]], dense[np.nonzero(kept)[0] // w.top_k])


def test_ffn_rows_outside_segments_untouched():
    w, idx, wts, lay, x, xp, wgu, wd = _small_ffn_case()
    rows = np.array([lay["rows"] - 1, 0], np.int64)
    lay2 = dict(lay)
    lay2["tokens_per_expert"] = lay["tokens_per_expert"].copy()
    lay2["tokens_per_expert"][-1] = max(0, lay2["tokens_per_expert"][-1] - 1)
    _, ex = oracle.expert_ffn_rows(rows, xp, lay2, wgu, wd)
    assert ex[0] == -1 and ex[1] >= 0


# ------------------------------------------------------- expert FFN backward

def _ffn_forward_f64(x, wgu, wd, lay):
    """Independent fp64 forward of the grouped SwiGLU FFN (no rounding)."""
    e, two_i, _ = wgu.shape
    inter = two_i // 2
    y = np.zeros((x.shape[0], wd.shape[1]))
    for ex in range(e):
        o, n = int(lay["expert_offsets"][ex]), int(lay["tokens_per_expert"][ex])
        for r in range(o, o + n):
            gv = wgu[ex, :inter] @ x[r]
            uv = wgu[ex, inter:] @ x[r]
            y[r] = wd[ex] @ (gv / (1.0 + np.exp(-gv)) * uv)
    return y


def _ffn_bwd_case(seed=5, capacity=0):
    g = np.random.default_rng(seed)
    n, k, e, h, inter = 9, 2, 3, 8, 4
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    idx[0, :] = [0, 2]
    idx[:, :][idx == 1] = 0            # expert 1 receives no rows
    lay = oracle.layout(idx, e, capacity)
    x = g.standard_normal((lay["rows"], h))
    wgu = g.standard_normal((e, 2 * inter, h)) * 0.5
    wd = g.standard_normal((e, h, inter)) * 0.5
    dy = g.standard_normal((lay["rows"], h))
    return lay, x, wgu, wd, dy


def test_ffn_bwd_central_finite_differences():
    lay, x, wgu, wd, dy = _ffn_bwd_case()
    gx, dwgu, dwd = oracle.expert_ffn_bwd(x, dy, lay, wgu, wd, round_out=False)
    loss = lambda x_, wgu_, wd_: (_ffn_forward_f64(x_, wgu_, wd_, lay) * dy).sum()
    g = np.random.default_rng(6)
    eps = 1e-6
    in_seg = np.nonzero(lay["pad_mask"] == 0)[0]
    checks = []
    for _ in range(12):                # inputs: rows of the segments
        r, c = int(g.choice(in_seg)), int(g.integers(x.shape[1]))
        xp, xm = x.copy(), x.copy()
        xp[r, c] += eps
        xm[r, c] -= eps
        checks.append(((loss(xp, wgu, wd) - loss(xm, wgu, wd)) / (2 * eps), gx[r, c]))
    for _ in range(12):                # gate and up weights of experts 0 and 2
        ex, i, c = int(g.choice([0, 2])), int(g.integers(wgu.shape[1])), int(g.integers(wgu.shape[2]))
        wp, wm = wgu.copy(), wgu.copy()
        wp[ex, i, c] += eps
        wm[ex, i, c] -= eps
        checks.append(((loss(x, wp, wd) - loss(x, wm, wd)) / (2 * eps), dwgu[ex, i, c]))
    for _ in range(12):                # down weights
        ex, i, c = int(g.choice([0, 2])), int(g.integers(wd.shape[1])), int(g.integers(wd.shape[2]))
        wp, wm = wd.copy(), wd.copy()
        wp[ex, i, c] += eps
        wm[ex, i, c] -= eps
        checks.append(((loss(x, wgu, wp) - loss(x, wgu, wm)) / (2 * eps), dwd[ex, i, c]))
    for fd, an in checks:
        assert abs(fd - an) <= 1e-6 * (1 + abs(fd)), (fd, an)


def test_ffn_bwd_euler_in_down_weights_and_empty_expert():
    lay, x, wgu, wd, dy = _ffn_bwd_case(7)
    gx, dwgu, dwd = oracle.expert_ffn_bwd(x, dy, lay, wgu, wd, round_out=False)
    # y is linear in W_down: <grad W_down, W_down> = <dY, Y>
    y = _ffn_forward_f64(x, wgu, wd, lay)
    assert abs((dwd * wd).sum() - (dy * y).sum()) <= 1e-9 * (np.abs(dy * y).sum() + 1)
    assert lay["tokens_per_expert"][1] == 0
    assert (dwgu[1] == 0).all() and (dwd[1] == 0).all()
    outside = lay["pad_mask"] != 0
    assert (gx[outside] == 0).all()


def test_ffn_bwd_rounding_is_one_rne_per_value():
    lay, x, wgu, wd, dy = _ffn_bwd_case(8)
    exact = oracle.expert_ffn_bwd(x, dy, lay, wgu, wd, round_out=False)
    rounded = oracle.expert_ffn_bwd(x, dy, lay, wgu, wd)
    for a, b in zip(exact, rounded):
        a, b = a.reshape(-1), b.reshape(-1)
        nz = a != 0                    # the reference rounding covers the normal range
        assert (bf16_from_double_ref(a[nz]) == b[nz]).all()
        assert (b[~nz] & 0x7FFF == 0).all()


def test_ffn_bwd_entries_match_the_whole_backward():
    """The per-entry backward used at full sizes agrees with the whole-matrix one
    (itself pinned by finite differences above) on bf16 inputs."""
    lay, x, wgu, wd, dy = _ffn_bwd_case(9)
    bits = lambda a: mi.f32_to_bf16_bits(a.astype(np.float32))
    x, wgu, wd, dy = bits(x), bits(wgu * 0.2), bits(wd * 0.2), bits(dy)
    gx, dwgu, dwd = oracle.expert_ffn_bwd(x, dy, lay, wgu, wd)
    rows = np.nonzero(lay["pad_mask"] == 0)[0]
    e, two_i, h = wgu.shape
    dwd_idx = [(ex, hh, i) for ex in range(e) for hh in range(h) for i in range(two_i // 2)]
    dwgu_idx = [(ex, j, hh) for ex in range(e) for j in range(two_i) for hh in range(h)]
    g_rows, g_dwd, g_dwgu = oracle.expert_ffn_bwd_entries(x, dy, lay, wgu, wd, rows, dwd_idx, dwgu_idx)
    pairs = [(g_rows, gx[rows]), (g_dwd, np.array([dwd[i] for i in dwd_idx])),
             (g_dwgu, np.array([dwgu[i] for i in dwgu_idx]))]
    for got, ref in pairs:
        got, ref = got.reshape(-1).astype(np.int32), ref.reshape(-1).astype(np.int32)
        assert (np.abs(got - ref) <= 1).all()      # fp64 sums in another order: at most one bf16 step apart
        assert (got == ref).mean() > 0.98


def test_gate_up_rows_brute_force():
    """Pre-activations by plain Python loops over a tiny case."""
    g = np.random.default_rng(12)
    e, h, inter = 3, 8, 4
    idx = np.array([[0, 2], [1, 2], [2, 0], [0, 1]], np.int32)
    lay = oracle.layout(idx, e)
    x = mi.f32_to_bf16_bits(g.standard_normal((lay["rows"], h)).astype(np.float32))
    wgu = mi.f32_to_bf16_bits((g.standard_normal((e, 2 * inter, h)) * 0.3).astype(np.float32))
    rows = list(range(lay["rows"]))
    got = oracle.expert_gate_up_rows(rows, x, lay, wgu)
    xv, wv = bf16_vals(x), bf16_vals(wgu)
    for n, r in enumerate(rows):
        ex = next(q for q in range(e) if lay["expert_offsets"][q] <= r < lay["expert_offsets"][q] + lay["tokens_per_expert"][q])
        ref = [sum(float(xv[r, c]) * float(wv[ex, i, c]) for c in range(h)) for i in range(2 * inter)]
        assert (got[n] == bf16_from_double_ref(np.array(ref))).all()
