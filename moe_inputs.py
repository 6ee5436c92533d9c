"""Seeded synthetic inputs for the single-GPU MoE dispatch -> expert -> combine path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It draws random numbers and arranges them into the shapes and
structures of the five workloads below; it computes none of the method itself
(no softmax, no top-k result, no layout, no combine).  The only selection it
performs is inside the Zipf-bias calibration of the skewed workload, where a
library partial sort (numpy.argpartition) is used to measure how loads respond
to a bias while the bias is tuned; the result of that calibration is an input
(a logit offset per expert), never an expected output.

Workloads (sizes from the dispatch/combine validation shape reported on the
mscclpp "high-throughput MoE dispatch/combine" commit page: 4096 tokens, hidden
7168, 256 experts, top-8; the expert-FFN shapes follow the Qwen3-235B-A22B and
DeepSeek-V3 model families named on the Megatron-LM "Add MORI as a Token
Dispatcher" and xtuner "Integrate UltraEP Runtime" pages):

  tiny            N=64 H=128 E=8 k=2 fp32, identity expert
  uniform         N=4096 H=7168 E=256 k=8 bf16, N(0,1) logits, identity expert
  zipf_capacity   as uniform, logits + per-expert bias giving Zipf(1.2) loads,
                  capacity factor 1.25, identity expert
  qwen3_layer     N=8192 H=4096 E=128 k=8, SwiGLU experts with I=1536
  dsv3_share      32 local experts, H=7168, I=2048, 16384 received tokens with
                  8 slots each (2 local ids, 6 sentinel -1), 32768 rows whose
                  per-expert counts follow Zipf(1.2)

Random streams: numpy default_rng(SeedSequence([workload_id, stream, ...])),
stream 0 = logits, 1 = activations, 2 = gate/up weights, 3 = down weights,
4 = output gradient, 5 = routing construction.  bf16 tensors are the
round-to-nearest-even bf16 values of fp32 N(0, std) draws, stored as uint16 bit
patterns.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

STREAM_LOGITS = 0
STREAM_X = 1
STREAM_W_GATE_UP = 2
STREAM_W_DOWN = 3
STREAM_GRAD = 4
STREAM_ROUTING = 5
STREAM_GRAD_ROWS = 6

DT_F32 = 0
DT_BF16 = 1


@dataclass(frozen=True)
class Workload:
    wid: int                 # workload id (1..5), the first seed word
    name: str
    n_tokens: int            # N (received tokens for dsv3_share)
    hidden: int              # H
    n_experts: int           # E (local experts)
    top_k: int               # k slots per token
    dtype: int               # DT_F32 or DT_BF16 activations
    inter: int = 0           # I, SwiGLU intermediate size (0 = identity expert)
    capacity_factor: float = 0.0
    zipf_s: float = 0.0      # Zipf exponent for skewed loads (0 = none)
    rows: int = 0            # dsv3_share: number of valid rows (local assignments)
    local_per_token: int = 0  # dsv3_share: local ids per received token
    has_router: bool = True
    backward: bool = False
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def capacity(self) -> int:
        """Per-expert capacity C = ceil(cf * N * k / E); 0 means dropless."""
        if self.capacity_factor <= 0:
            return 0
        return int(math.ceil(self.capacity_factor * self.n_tokens * self.top_k / self.n_experts - 1e-9))

    @property
    def max_rows(self) -> int:
        if self.capacity:
            return self.n_experts * self.capacity
        if self.rows:
            return self.rows
        return self.n_tokens * self.top_k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DT_F32 else 2


WORKLOADS = {
    1: Workload(1, "tiny", 64, 128, 8, 2, DT_F32),
    2: Workload(2, "uniform", 4096, 7168, 256, 8, DT_BF16),
    3: Workload(3, "zipf_capacity", 4096, 7168, 256, 8, DT_BF16, capacity_factor=1.25, zipf_s=1.2),
    4: Workload(4, "qwen3_layer", 8192, 4096, 128, 8, DT_BF16, inter=1536),
    5: Workload(5, "dsv3_share", 16384, 7168, 32, 8, DT_BF16, inter=2048, zipf_s=1.2,
                rows=32768, local_per_token=2, has_router=False, backward=True),
}


def workload(wid: int, **overrides) -> Workload:
    """The workload `wid`, optionally with shapes overridden (for scaled-down tests)."""
    w = WORKLOADS[wid]
    return replace(w, **overrides) if overrides else w


def _rng(*words: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(v) for v in words]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_activations(shape, dtype: int, *seed_words, std: float = 1.0, threads: int = 8) -> np.ndarray:
    """N(0, std^2) activations; fp32 array or bf16 bit patterns (uint16).

    Large tensors are drawn in row blocks, each from its own sub-stream, so the
    values do not depend on the thread count.
    """
    shape = tuple(int(s) for s in shape)
    rows = shape[0]
    cols = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, cols), dtype=np.float32 if dtype == DT_F32 else np.uint16)
    block = max(1, (1 << 22) // max(cols, 1))

    def fill(b0):
        b1 = min(rows, b0 + block)
        g = _rng(*seed_words, b0 // block)
        v = g.standard_normal((b1 - b0, cols), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[b0:b1] = v if dtype == DT_F32 else f32_to_bf16_bits(v)

    starts = list(range(0, rows, block))
    if len(starts) > 1 and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, starts))
    else:
        for s in starts:
            fill(s)
    return out.reshape(shape)


def zipf_targets(n_experts: int, total: int, s: float, cap: int) -> np.ndarray:
    """Zipf(s) loads over experts (expert 0 hottest), summing to `total`, each capped
    at `cap` (a token cannot pick one expert twice), excess water-filled onto the
    rest, rounded by largest remainder."""
    w = 1.0 / np.arange(1, n_experts + 1, dtype=np.float64) ** s
    fixed = np.zeros(n_experts, dtype=bool)
    t = np.zeros(n_experts)
    for _ in range(n_experts):
        free = ~fixed
        rem = total - cap * fixed.sum()
        t[free] = rem * w[free] / w[free].sum()
        t[fixed] = cap
        over = free & (t > cap)
        if not over.any():
            break
        fixed |= over
    base = np.floor(t).astype(np.int64)
    short = int(total - base.sum())
    if short > 0:
        order = np.argsort(-(t - base), kind="stable")
        base[order[:short]] += 1
    return base


def _topk_loads(logits: np.ndarray, k: int) -> np.ndarray:
    sel = np.argpartition(-logits, k - 1, axis=1)[:, :k]
    return np.bincount(sel.ravel(), minlength=logits.shape[1])


def zipf_bias(z: np.ndarray, k: int, s: float, rounds: int = 120) -> np.ndarray:
    """A per-expert logit bias b (fp32) such that top-k of (z + b) gives loads close to
    the capped Zipf(s) targets.  Deterministic given z."""
    n, e = z.shape
    target = zipf_targets(e, n * k, s, n).astype(np.float64)
    b = np.log(np.maximum(target, 0.5) / (n * k / e))
    best, best_err = b.copy(), np.inf
    for _ in range(rounds):
        loads = _topk_loads(z + b.astype(np.float32), k)
        err = np.abs(loads - target).sum()
        if err < best_err:
            best, best_err = b.copy(), err
        b = b + 0.3 * (np.log(target + 0.5) - np.log(loads + 0.5))
    return best.astype(np.float32)


def router_logits(w: Workload, seed: int = 0) -> np.ndarray:
    """fp32 router logits [N, E]: N(0,1), plus the calibrated Zipf bias when skewed."""
    z = _rng(w.wid, STREAM_LOGITS, seed).standard_normal((w.n_tokens, w.n_experts), dtype=np.float32)
    if w.zipf_s > 0 and w.has_router:
        z = (z + zipf_bias(z, w.top_k, w.zipf_s)[None, :]).astype(np.float32)
    return np.ascontiguousarray(z)


def received_routing(w: Workload, seed: int = 0):
    """dsv3_share token structure: topk_idx int32 [T, k] with `local_per_token` local
    expert ids per token (others -1) and exact Zipf(s) per-expert counts summing to
    `rows`; topk_w fp32 [T, k] = softmax of N(0,1) draws over all k slots (the local
    pair therefore sums to < 1, as on the receiving rank of an expert-parallel
    dispatch)."""
    t, k, e = w.n_tokens, w.top_k, w.n_experts
    lp = w.local_per_token
    assert w.rows == t * lp
    counts = zipf_targets(e, w.rows, w.zipf_s, t)
    assert counts.max() < t
    g = _rng(w.wid, STREAM_ROUTING, seed)
    sorted_ids = np.repeat(np.arange(e, dtype=np.int32), counts)       # expert-sorted list
    per_token = sorted_ids.reshape(lp, t).T                             # token i gets L[i], L[i+T], ...
    order = g.permutation(t)                                            # shuffle token ids
    idx = np.full((t, k), -1, dtype=np.int32)
    for tok_pos in range(t):
        slots = g.choice(k, size=lp, replace=False)
        idx[order[tok_pos], slots] = per_token[tok_pos]
    r = g.standard_normal((t, k))
    r = np.exp(r - r.max(axis=1, keepdims=True))
    wts = (r / r.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, wts


def expert_weights(w: Workload, seed: int = 0, threads: int = 8):
    """bf16 SwiGLU weights: w_gate_up [E, 2I, H] (gate rows 0..I-1, up rows I..2I-1)
    and w_down [E, H, I], N(0, 0.02^2), one sub-stream per expert."""
    e, h, i = w.n_experts, w.hidden, w.inter
    wgu = np.empty((e, 2 * i, h), dtype=np.uint16)
    wd = np.empty((e, h, i), dtype=np.uint16)

    def one(ex):
        wgu[ex] = f32_to_bf16_bits(_rng(w.wid, STREAM_W_GATE_UP, seed, ex).standard_normal((2 * i, h), dtype=np.float32) * np.float32(0.02))
        wd[ex] = f32_to_bf16_bits(_rng(w.wid, STREAM_W_DOWN, seed, ex).standard_normal((h, i), dtype=np.float32) * np.float32(0.02))

    if threads > 1 and e > 1:
        with ThreadPoolExecutor(threads) as ex_:
            list(ex_.map(one, range(e)))
    else:
        for ex in range(e):
            one(ex)
    return wgu, wd


def activations(w: Workload, seed: int = 0) -> np.ndarray:
    return normal_activations((w.n_tokens, w.hidden), w.dtype, w.wid, STREAM_X, seed)


def grad_output(w: Workload, seed: int = 0) -> np.ndarray:
    return normal_activations((w.n_tokens, w.hidden), w.dtype, w.wid, STREAM_GRAD, seed)


def grad_expert_rows(w: Workload, rows: int, seed: int = 0) -> np.ndarray:
    """Incoming gradient of the expert outputs: bf16 [rows, H] ~ N(0, 1)."""
    return normal_activations((rows, w.hidden), DT_BF16, w.wid, STREAM_GRAD_ROWS, seed)
