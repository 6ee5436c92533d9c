"""Pins for the oracle's hot-expert replication (placement, reroute, replica
weight sync, replica gradient reduce).  CPU only.

Source: InternLM/xtuner pull request "Integrate UltraEP Runtime" (replicas of
hot experts from the current load, part of their tokens rerouted to replica
slots, master/replica weight sync, replica gradients reduced into the masters).
Readings checked here: slots are filled one at a time, each to the expert with
the largest load per copy (ties to the lower id); an expert's assignments are cut,
in assignment order, into 1 + slots consecutive runs as equal as possible, run j
holding the ordinals o with floor(o * m / c) = j.

Pins: exhaustive search over every allocation of the slots on small cases (the
greedy placement attains the smallest possible largest load per copy), closed
forms (equal loads go round robin, a single hot expert takes every slot), a
hand-worked reroute, a brute force of the runs from the floor formula, run-size
invariants, numpy fancy indexing for the weight sync and exact small-integer
sums for the gradient reduce.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import moe_inputs as mi
import oracle

RNG = np.random.default_rng(4242)


def allocations(e: int, r: int):
    for cut in itertools.combinations_with_replacement(range(e), r):
        yield np.bincount(np.array(cut, dtype=np.int64), minlength=e)


@pytest.mark.parametrize("seed", range(40))
def test_plan_minimises_the_largest_load_per_copy(seed):
    g = np.random.default_rng(seed)
    e, r = int(g.integers(1, 6)), int(g.integers(0, 6))
    counts = g.integers(0, 50, e).astype(np.int32)
    if seed % 4 == 0:
        counts[:] = counts[0]                           # all equal
    rep = oracle.replica_plan(counts, r)
    assert rep.shape == (r,) and ((rep >= 0) & (rep < e)).all()
    slots = np.bincount(rep, minlength=e)
    got = max(c / (1 + s) for c, s in zip(counts, slots))
    best = min(max(c / (1 + s) for c, s in zip(counts, a)) for a in allocations(e, r))
    assert got == best
    # slot i went to an expert with the largest load per copy at that moment, lowest id first
    taken = np.zeros(e, np.int64)
    for x in rep:
        loads = counts / (1 + taken)
        assert loads[x] == loads.max() and x == int(np.argmax(loads))
        taken[x] += 1


def test_plan_closed_forms():
    assert oracle.replica_plan(np.array([7, 7, 7]), 5).tolist() == [0, 1, 2, 0, 1]
    assert oracle.replica_plan(np.array([0, 90, 3, 4]), 3).tolist() == [1, 1, 1]
    assert oracle.replica_plan(np.array([0, 0, 0]), 2).tolist() == [0, 0]
    assert oracle.replica_plan(np.array([10, 40, 40, 5]), 4).tolist() == [1, 2, 1, 2]
    assert oracle.replica_plan(np.array([5, 9]), 0).size == 0


def test_reroute_hand_worked():
    """E = 4, slots [1, 2, 1]: expert 1 has 6 assignments in 3 runs of 2 (master,
    slot 0 = physical 4, slot 2 = physical 6); expert 2 has 2 in 2 runs (master,
    slot 1 = physical 5); -1 stays, the invalid id 7 becomes -2."""
    idx = np.array([[1, 2], [1, 0], [1, 3], [2, 1], [1, -1], [7, 1]], np.int32)
    got = oracle.reroute(idx, 4, np.array([1, 2, 1]))
    assert got.tolist() == [[1, 2], [1, 0], [4, 3], [5, 4], [6, -1], [-2, 6]]


def bf_reroute(idx: np.ndarray, e: int, rep: np.ndarray) -> np.ndarray:
    flat = idx.reshape(-1)
    out = np.where(flat == -1, -1, -2).astype(np.int32)
    for x in range(e):
        pos = np.nonzero(flat == x)[0]
        slots = [i for i in range(rep.size) if rep[i] == x]
        m, c = 1 + len(slots), pos.size
        for o, a in enumerate(pos):
            run = o * m // c
            out[a] = x if run == 0 else e + slots[run - 1]
    return out.reshape(idx.shape)


@pytest.mark.parametrize("seed", range(30))
def test_reroute_brute_force_and_run_sizes(seed):
    g = np.random.default_rng(100 + seed)
    n, e, k = int(g.integers(1, 300)), int(g.integers(1, 40)), 1 + seed % 4
    k = min(k, e)
    idx = np.stack([g.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if seed % 3 == 0:
        idx[g.random(idx.shape) < 0.1] = -1
    if seed % 5 == 0:
        idx[g.random(idx.shape) < 0.05] = g.choice([-7, e, e + 3])
    counts = np.bincount(idx[(idx >= 0) & (idx < e)], minlength=e).astype(np.int32)
    r = int(g.integers(0, 2 * e + 1))
    rep = oracle.replica_plan(counts, r)
    got = oracle.reroute(idx, e, rep)
    np.testing.assert_array_equal(got, bf_reroute(idx, e, rep))
    # every copy of an expert gets floor or ceil of count / copies, the master the ceil;
    # the physical counts of an expert's copies add up to its count
    phys_counts = np.bincount(got[got >= 0], minlength=e + r)
    for x in range(e):
        copies = [x] + [e + i for i in range(r) if rep[i] == x]
        c, m = counts[x], len(copies)
        sizes = phys_counts[copies]
        assert sizes.sum() == c and sizes.max() - sizes.min() <= 1 and sizes[0] == -(-c // m)
    # assignment order is kept within each physical expert, and the runs follow each other
    flat = got.reshape(-1)
    for x in range(e):
        pos = np.nonzero(idx.reshape(-1) == x)[0]
        copies = [x] + [e + i for i in range(r) if rep[i] == x]
        order = [copies.index(p) for p in flat[pos]]
        assert order == sorted(order)


def test_reroute_then_layout_keeps_every_token():
    """The layout over the physical ids keeps each assignment once; the logical
    expert of every placed row is the one the router chose."""
    w = mi.workload(2, n_tokens=512)
    idx, _, _, _ = oracle.route(mi.router_logits(w), w.top_k)
    counts = np.bincount(idx.reshape(-1), minlength=w.n_experts)
    rep = oracle.replica_plan(counts, 16)
    phys = oracle.reroute(idx, w.n_experts, rep)
    lay = oracle.layout(phys, w.n_experts + 16)
    assert lay["counters"][0] == idx.size and lay["counters"][1] == 0
    logical_of = np.concatenate([np.arange(w.n_experts), rep])
    placed = lay["row_src"] >= 0
    src = lay["row_src"][placed]
    assert (logical_of[phys.reshape(-1)[src]] == idx.reshape(-1)[src]).all()


def test_replica_sync_and_grad_reduce():
    e, r, shape = 6, 5, (3, 8)
    rep = np.array([2, 4, 2, 0, 2], np.int32)
    master = mi.f32_to_bf16_bits(RNG.standard_normal((e,) + shape).astype(np.float32))
    np.testing.assert_array_equal(oracle.replica_sync(master, rep), master[rep])
    # small integers: every sum is exact, so the reduce is plain addition
    gm = RNG.integers(-50, 50, (e,) + shape).astype(np.float32)
    gr = RNG.integers(-50, 50, (r,) + shape).astype(np.float32)
    got = oracle.replica_grad_reduce(mi.f32_to_bf16_bits(gm), mi.f32_to_bf16_bits(gr), rep)
    want = gm.copy()
    np.add.at(want, rep, gr)
    np.testing.assert_array_equal(mi.bf16_bits_to_f32(got), want)
    # general values: one rounding of the exact sum, experts without slots untouched
    gm = mi.f32_to_bf16_bits(RNG.standard_normal((e,) + shape).astype(np.float32))
    gr = mi.f32_to_bf16_bits(RNG.standard_normal((r,) + shape).astype(np.float32))
    got = oracle.replica_grad_reduce(gm, gr, rep)
    exact = mi.bf16_bits_to_f32(gm).astype(np.float64)
    np.add.at(exact, rep, mi.bf16_bits_to_f32(gr).astype(np.float64))
    np.testing.assert_array_equal(got[[0, 2, 4]], oracle.bf16_round_array(exact[[0, 2, 4]]))
    np.testing.assert_array_equal(got[[1, 3, 5]], gm[[1, 3, 5]])
