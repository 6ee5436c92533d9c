"""CPU oracle for the single-GPU MoE route -> dispatch -> expert FFN -> combine path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's cpu_baseline leg, never by the product package.  It wraps the plain
C reference in moe_oracle.c (fp64 arithmetic except where a step fixes another
precision; see that file's header for the sources of each step) and shares no
code with the GPU library.

Every oracle function here is pinned by the CPU tests in tests/test_oracle_pins.py
against brute force on tiny inputs, closed forms and invariants.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "moe_oracle.c"
# MOE_ORACLE_SANITIZE=1: a separate build with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only; the process must preload the
# ASan runtime), for running the pins under the sanitizers
_SANITIZE = os.environ.get("MOE_ORACLE_SANITIZE") == "1"
_LIB = _HERE / ("libmoe_oracle_san.so" if _SANITIZE else "libmoe_oracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

DT_F32 = 0
DT_BF16 = 1


def build(force: bool = True) -> Path:
    """Compile moe_oracle.c with gcc (plain C11, -O2, no floating-point contraction)."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                               *(_SAN_FLAGS if _SANITIZE else []), "-shared", "-o", str(tmp), str(_SRC), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        L = C.CDLL(str(_LIB))
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.oracle_route.argtypes = [i64, i32, i32, p, p, p, p, p, p, p]
        L.oracle_route.restype = i32
        L.oracle_philox4x32_10.argtypes = [p, p, p]
        L.oracle_philox4x32_10.restype = None
        L.oracle_random_logits.argtypes = [i64, i32, C.c_uint64, p]
        L.oracle_random_logits.restype = None
        L.oracle_layout_rows.argtypes = [i64, i32, i32, i32, i64, i32]
        L.oracle_layout_rows.restype = i64
        L.oracle_layout.argtypes = [i64, i32, i32, i32, i64, i32, i32, p, p, p, p, p, p, p, p, p, p]
        L.oracle_layout.restype = i32
        L.oracle_scatter.argtypes = [i64, i32, i64, p, p, p, i64, p, i64, p, p]
        L.oracle_scatter.restype = None
        L.oracle_expert_ffn_rows.argtypes = [i64, p, i32, i64, i64, p, p, p, p, p, p, p]
        L.oracle_expert_ffn_rows.restype = None
        L.oracle_combine.argtypes = [i64, i32, i64, i32, p, p, p, p]
        L.oracle_combine.restype = None
        L.oracle_combine_bwd.argtypes = [i64, i32, i64, i32, p, p, p, p, i64, p, i64, p, p]
        L.oracle_dispatch_bwd.argtypes = [i64, i32, i64, i32, p, p, p]
        L.oracle_dispatch_bwd.restype = None
        L.oracle_combine_bwd.restype = None
        L.oracle_bf16_round.argtypes = [C.c_double]
        L.oracle_bf16_round_array.argtypes = [i64, p, p]
        L.oracle_bf16_round_array.restype = None
        L.oracle_bf16_round.restype = C.c_uint16
        L.oracle_mx_quantize.argtypes = [i64, i64, p, p, p]
        L.oracle_expert_ffn_mxfp8_rows.argtypes = [i64, p, i32, i64, i64, p, p, p, p, p, p, p, p, p, p]
        L.oracle_expert_ffn_mxfp8_rows.restype = None
        L.oracle_replica_plan.argtypes = [i32, p, i32, p]
        L.oracle_replica_plan.restype = None
        L.oracle_reroute.argtypes = [i64, i32, i32, p, i32, p, p]
        L.oracle_reroute.restype = None
        L.oracle_replica_sync.argtypes = [i32, p, i64, p, p]
        L.oracle_replica_sync.restype = None
        L.oracle_replica_grad_reduce.argtypes = [i32, i32, p, i64, p, p]
        L.oracle_replica_grad_reduce.restype = None
        L.oracle_mx_quantize.restype = None
        L.oracle_e4m3_encode_array.argtypes = [i64, p, p]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_decode_array.argtypes = [i64, p, p]
        L.oracle_e4m3_decode_array.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return DT_F32
    if a.dtype == np.uint16:
        return DT_BF16
    raise TypeError(f"activations must be float32 or bf16 bits (uint16), got {a.dtype}")


def route(logits: np.ndarray, k: int, token_mask=None, expert_bias=None):
    """-> topk_idx int32 [N,k], topk_w fp32 [N,k], routing_map uint8 [N,E], tokens_per_expert int32 [E].
    token_mask (uint8 [N], optional): nonzero marks a padding token, routed nowhere (-1 slots, weight 0).
    expert_bias (fp32 [E], optional): selection-only bias (rank by logit + bias, weights from the logits)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    n, e = logits.shape
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float32)
    rmap = np.empty((n, e), np.uint8)
    tpe = np.empty(e, np.int32)
    mask = None if token_mask is None else np.ascontiguousarray(token_mask, dtype=np.uint8)
    assert mask is None or mask.shape == (n,)
    bias = None if expert_bias is None else np.ascontiguousarray(expert_bias, dtype=np.float32)
    assert bias is None or bias.shape == (e,)
    rc = lib().oracle_route(n, e, k, _p(logits), _p(bias), _p(mask), _p(idx), _p(w), _p(rmap), _p(tpe))
    if rc != 0:
        raise ValueError(f"oracle_route: bad arguments (rc={rc})")
    return idx, w, rmap, tpe


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon et al., SC 2011) of one counter (4 words) and key (2 words)."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def random_logits(n: int, e: int, seed: int) -> np.ndarray:
    """The force-balanced mode's router logits, fp32 [N, E] uniform in [0, 1) (moe_oracle.c)."""
    out = np.empty((n, e), np.float32)
    lib().oracle_random_logits(n, e, seed, _p(out))
    return out


def route_random(n: int, e: int, k: int, seed: int, token_mask=None, expert_bias=None):
    """Force-balanced routing: route() over random_logits(n, e, seed)."""
    return route(random_logits(n, e, seed), k, token_mask, expert_bias)


def layout(topk_idx: np.ndarray, n_experts: int, capacity: int = 0, max_rows: int = 0, row_align: int = 0,
           drop_policy: int = 0, topk_w=None) -> dict:
    """Dispatch layout; returns a dict of numpy arrays (see moe_oracle.c oracle_layout).
    drop_policy 1 (capacity only) keeps each expert's C largest weights topk_w."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    w = None if topk_w is None else np.ascontiguousarray(topk_w, dtype=np.float32)
    if drop_policy == 1 and capacity > 0:
        assert w is not None and w.shape == topk_idx.shape
    n, k = topk_idx.shape
    rows = lib().oracle_layout_rows(n, k, n_experts, capacity, max_rows, row_align)
    out = dict(
        tokens_per_expert=np.empty(n_experts, np.int32),
        expert_offsets=np.empty(n_experts + 1, np.int32),
        ordinal=np.empty(n * k, np.int32),
        assign_row=np.empty(n * k, np.int32),
        row_src=np.empty(rows, np.int32),
        drop_mask=np.empty(n * k, np.uint8),
        pad_mask=np.empty(rows, np.uint8),
        counters=np.empty(4, np.int32),
    )
    rc = lib().oracle_layout(n, k, n_experts, capacity, max_rows, row_align, drop_policy, _p(topk_idx), _p(w),
                             *[_p(out[f]) for f in ("tokens_per_expert", "expert_offsets", "ordinal",
                                                    "assign_row", "row_src", "drop_mask", "pad_mask", "counters")])
    if rc != 0:
        raise ValueError(f"oracle_layout: bad arguments (rc={rc})")
    out["rows"] = int(rows)
    return out


def scatter(x: np.ndarray, k: int, lay: dict, topk_w: np.ndarray, x_perm=None):
    """Permuted rows and weights: -> (x_perm [rows, H], w_perm [rows]).  Pad rows (below
    the end of the last segment, holding nothing) are zero; rows of an unused dropless
    tail keep what `x_perm` held (zeros if not given)."""
    x = np.ascontiguousarray(x)
    n, h = x.shape
    rows = lay["rows"]
    if x_perm is None:
        x_perm = np.zeros((rows, h), x.dtype)
    w_perm = np.empty(rows, np.float32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    lib().oracle_scatter(n, k, h * x.itemsize, _p(x), _p(lay["assign_row"]), _p(topk_w), rows,
                         _p(lay["row_src"]), int(lay["expert_offsets"][-1]), _p(x_perm), _p(w_perm))
    return x_perm, w_perm


def mx_quantize(x: np.ndarray):
    """MXFP8 of bf16 rows (uint16 bits [n, H], H % 32 == 0) -> (q uint8 [n, H] E4M3
    codes, scale uint8 [n, H/32] E8M0 codes); the OCP MX v1.0 conversion."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n, h = x.shape
    if h % 32:
        raise ValueError("row length must be a multiple of 32")
    q = np.empty((n, h), np.uint8)
    sc = np.empty((n, h // 32), np.uint8)
    lib().oracle_mx_quantize(n, h, _p(x), _p(q), _p(sc))
    return q, sc


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """double -> E4M3 codes (clamped to +-448, nearest, ties to even), element-wise."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_array(v.size, _p(v), _p(out))
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_array(c.size, _p(c), _p(out))
    return out


def mx_dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Values of MXFP8 rows: E4M3 value times 2^(scale code - 127), float64."""
    q = np.asarray(q, np.uint8)
    n, h = q.shape
    s = np.repeat(np.asarray(scale, np.int64).reshape(n, h // 32) - 127, 32, axis=1)
    return np.ldexp(e4m3_decode(q), s)


def expert_ffn_mxfp8_rows(rows, xq, xs, lay, wguq, wgus, wdq, wds):
    """SwiGLU FFN over MXFP8 operands for the listed permuted rows -> (y_rows bf16 bits [len, H],
    expert_of).  xq [R, H] / xs [R, H/32]; wguq [E, 2I, H] / wgus [E, 2I, H/32]; wdq [E, H, I] /
    wds [E, H, I/32]."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    e, two_i, h = wguq.shape
    inter = two_i // 2
    assert wdq.shape == (e, h, inter) and wgus.shape == (e, two_i, h // 32) and wds.shape == (e, h, inter // 32)
    y = np.zeros((rows.size, h), np.uint16)
    ex = np.empty(rows.size, np.int32)
    c = np.ascontiguousarray
    lib().oracle_expert_ffn_mxfp8_rows(rows.size, _p(rows), e, h, inter, _p(c(xq, dtype=np.uint8)),
                                       _p(c(xs, dtype=np.uint8)), _p(lay["expert_offsets"]),
                                       _p(lay["tokens_per_expert"]), _p(c(wguq, dtype=np.uint8)),
                                       _p(c(wgus, dtype=np.uint8)), _p(c(wdq, dtype=np.uint8)),
                                       _p(c(wds, dtype=np.uint8)), _p(y), _p(ex))
    return y, ex


def dispatch_mxfp8(x: np.ndarray, k: int, lay: dict, topk_w: np.ndarray, x_perm_q=None, x_perm_scale=None):
    """MXFP8 dispatch: each token row quantised (mx_quantize), then its codes and
    scales permuted like scatter() permutes bf16 rows -> (x_perm_q [rows, H],
    x_perm_scale [rows, H/32], w_perm [rows]); pad rows are all-zero bytes."""
    q, sc = mx_quantize(x)
    pq, w_perm = scatter(q, k, lay, topk_w, x_perm_q)
    ps, _ = scatter(sc, k, lay, topk_w, x_perm_scale)
    return pq, ps, w_perm


def replica_plan(counts: np.ndarray, r: int) -> np.ndarray:
    """Hot-expert placement: logical expert of each of r replica slots."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    out = np.empty(r, np.int32)
    lib().oracle_replica_plan(counts.size, _p(counts), r, _p(out))
    return out


def reroute(topk_idx: np.ndarray, n_experts: int, replica_of: np.ndarray) -> np.ndarray:
    """Logical -> physical expert ids [N, k] (physical E + i = replica slot i)."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    rep = np.ascontiguousarray(replica_of, dtype=np.int32)
    out = np.empty_like(idx)
    n, k = idx.shape
    lib().oracle_reroute(n, k, n_experts, _p(idx), rep.size, _p(rep), _p(out))
    return out


def replica_sync(master: np.ndarray, replica_of: np.ndarray) -> np.ndarray:
    """Replica weights [R, ...] copied from the masters [E, ...] (bf16 bits)."""
    master = np.ascontiguousarray(master, dtype=np.uint16)
    rep = np.ascontiguousarray(replica_of, dtype=np.int32)
    out = np.empty((rep.size,) + master.shape[1:], np.uint16)
    elems = int(np.prod(master.shape[1:]))
    lib().oracle_replica_sync(rep.size, _p(rep), elems, _p(master), _p(out))
    return out


def replica_grad_reduce(grad_master: np.ndarray, grad_replica: np.ndarray, replica_of: np.ndarray) -> np.ndarray:
    """Master gradients [E, ...] plus their replicas' [R, ...] (bf16 bits, one rounding)."""
    gm = np.ascontiguousarray(grad_master, dtype=np.uint16).copy()
    gr = np.ascontiguousarray(grad_replica, dtype=np.uint16)
    rep = np.ascontiguousarray(replica_of, dtype=np.int32)
    elems = int(np.prod(gm.shape[1:]))
    lib().oracle_replica_grad_reduce(gm.shape[0], rep.size, _p(rep), elems, _p(gr), _p(gm))
    return gm


def expert_ffn_rows(rows, x_perm, lay, w_gate_up, w_down):
    """SwiGLU FFN output rows (bf16 bits) for the listed permuted rows -> (y_rows [len, H], expert_of)."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    e, two_i, h = w_gate_up.shape
    inter = two_i // 2
    assert x_perm.dtype == np.uint16 and w_gate_up.dtype == np.uint16 and w_down.dtype == np.uint16
    assert w_down.shape == (e, h, inter)
    y = np.zeros((rows.size, h), np.uint16)
    ex = np.empty(rows.size, np.int32)
    lib().oracle_expert_ffn_rows(rows.size, _p(rows), e, h, inter, _p(np.ascontiguousarray(x_perm)),
                                 _p(lay["expert_offsets"]), _p(lay["tokens_per_expert"]),
                                 _p(np.ascontiguousarray(w_gate_up)), _p(np.ascontiguousarray(w_down)),
                                 _p(y), _p(ex))
    return y, ex


def expert_gate_up_rows(rows, x_perm, lay, w_gate_up):
    """Pre-activations of the listed permuted rows (rows inside the segments):
    [G | U][r, i] = bf16(x_perm[r] . w_gate_up[e, i]) for i < 2I, e the row's
    expert -- the first GEMM of the SwiGLU FFN before the activation.  fp64 dot
    products, one rounding.  -> bf16 bits [len(rows), 2I]."""
    e, two_i, h = w_gate_up.shape
    offs = [int(v) for v in lay["expert_offsets"][:e]]
    cnts = [int(v) for v in lay["tokens_per_expert"][:e]]
    out = np.zeros((len(rows), two_i))
    for n, r in enumerate(rows):
        ex = [x for x in range(e) if offs[x] <= int(r) < offs[x] + cnts[x]]
        if len(ex) != 1:
            raise ValueError(f"row {r} is not inside exactly one expert segment")
        out[n] = _bf16_f64(w_gate_up[ex[0]]) @ _bf16_f64(x_perm[r])
    return bf16_round_array(out)


def expert_ffn_segments(x_perm, lay, w_gate_up, w_down, experts=None):
    """The grouped SwiGLU FFN of oracle_expert_ffn_rows taken one expert segment
    at a time with fp64 matrix products (a library matmul: every product of two
    bf16 values is exact in fp64 and the sums are fp64, in the library's order
    rather than the C loop's) and the same two bf16 roundings:
        a = bf16(silu(x . w_gate) * (x . w_up)),  y = bf16(a . w_down),
    silu(z) = z / (1 + e^-z).  For full-size checks of every row, where the C
    loop takes too long.  Yields (expert, first row, y rows [count, H] as bf16
    bits) for every non-empty segment among `experts` (default: all)."""
    e, two_i, h = w_gate_up.shape
    inter = two_i // 2
    for ex in (range(e) if experts is None else experts):
        o, n = int(lay["expert_offsets"][ex]), int(lay["tokens_per_expert"][ex])
        if n == 0:
            continue
        x = _bf16_f64(x_perm[o:o + n])
        g = x @ _bf16_f64(w_gate_up[ex, :inter]).T
        u = x @ _bf16_f64(w_gate_up[ex, inter:]).T
        a = _bf16_f64(bf16_round_array(g / (1.0 + np.exp(-g)) * u))
        del g, u
        yield ex, o, bf16_round_array(a @ _bf16_f64(w_down[ex]).T)


def expert_ffn(x_perm, lay, w_gate_up, w_down):
    """FFN over every kept row; rows outside the segments are returned as zeros."""
    rows = np.nonzero(lay["pad_mask"] == 0)[0]
    y_rows, _ = expert_ffn_rows(rows, x_perm, lay, w_gate_up, w_down)
    y = np.zeros((lay["rows"], x_perm.shape[1]), np.uint16)
    y[rows] = y_rows
    return y


def combine(y: np.ndarray, topk_w: np.ndarray, lay: dict, n: int, k: int):
    y = np.ascontiguousarray(y)
    h = y.shape[1]
    out = np.empty((n, h), y.dtype)
    lib().oracle_combine(n, k, h, _dt(y), _p(y), _p(np.ascontiguousarray(topk_w, dtype=np.float32)),
                         _p(lay["assign_row"]), _p(out))
    return out


def dispatch_bwd(grad_x_perm: np.ndarray, lay: dict, n: int, k: int):
    """Adjoint of the row scatter: grad_x [N, H] = sum of the kept slots' rows."""
    grad_x_perm = np.ascontiguousarray(grad_x_perm)
    h = grad_x_perm.shape[1]
    out = np.empty((n, h), grad_x_perm.dtype)
    lib().oracle_dispatch_bwd(n, k, h, _dt(grad_x_perm), _p(grad_x_perm), _p(lay["assign_row"]), _p(out))
    return out


def combine_bwd(grad_out: np.ndarray, y: np.ndarray, topk_w: np.ndarray, lay: dict, k: int, grad_y=None):
    """-> (grad_y [rows, H], grad_w fp32 [N, k]).  Unused dropless tail rows keep what
    `grad_y` held (zeros if not given)."""
    grad_out = np.ascontiguousarray(grad_out)
    y = np.ascontiguousarray(y)
    n, h = grad_out.shape
    assert y.dtype == grad_out.dtype
    rows = lay["rows"]
    if grad_y is None:
        grad_y = np.zeros((rows, h), y.dtype)
    grad_w = np.empty((n, k), np.float32)
    lib().oracle_combine_bwd(n, k, h, _dt(y), _p(grad_out), _p(y),
                             _p(np.ascontiguousarray(topk_w, dtype=np.float32)), _p(lay["assign_row"]),
                             rows, _p(lay["row_src"]), int(lay["expert_offsets"][-1]), _p(grad_y), _p(grad_w))
    return grad_y, grad_w


def bf16_round_array(x: np.ndarray) -> np.ndarray:
    """double -> bf16 bits (round to nearest, ties to even), element-wise."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_round_array(x.size, _p(x), _p(out))
    return out


def _bf16_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 (exact: the bits are the top half of an fp32)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_ffn_bwd(x_perm, grad_y, lay, w_gate_up, w_down, round_out=True):
    """Backward of the grouped SwiGLU FFN, per expert segment (rows
    expert_offsets[e] .. + tokens_per_expert[e]) of the expert-contiguous buffer.

    With G = X Wg^T, U = X Wu^T, s = sigmoid(G), A = G s U, Y = A Wd^T and the
    incoming dY:
        dA = dY Wd,  dG = dA U s (1 + G (1 - s)),  dU = dA G s,
        dX = dG Wg + dU Wu,  dWd = dY^T A,  dWg = dG^T X,  dWu = dU^T X
    (the chain rule through y = Wd (silu(Wg x) * (Wu x)); silu'(g) = s(1 + g(1 - s))).
    fp64 numpy matmuls, no intermediate rounding.  Inputs are bf16 bits (or
    float64 arrays, used as they are).  Returns (grad_x_perm [R, H],
    grad_w_gate_up [E, 2I, H], grad_w_down [E, H, I]) as bf16 bits, each value
    rounded once (round_out=False: the float64 values).  Rows outside the
    segments of grad_x_perm are zero; experts without rows get zero gradients.
    """
    e, two_i, h = w_gate_up.shape
    inter = two_i // 2
    gx = np.zeros((lay["rows"], h))
    dwgu = np.zeros((e, two_i, h))
    dwd = np.zeros((e, h, inter))
    for ex in range(e):
        o, n = int(lay["expert_offsets"][ex]), int(lay["tokens_per_expert"][ex])
        if n == 0:
            continue
        gx[o:o + n], dwgu[ex], dwd[ex] = expert_ffn_bwd_expert(x_perm, grad_y, lay, w_gate_up, w_down, ex,
                                                               round_out=False)
    if not round_out:
        return gx, dwgu, dwd
    return bf16_round_array(gx), bf16_round_array(dwgu), bf16_round_array(dwd)


def expert_ffn_bwd_expert(x_perm, grad_y, lay, w_gate_up, w_down, ex, round_out=True):
    """expert_ffn_bwd for the one expert `ex` (the same formulas over its segment
    only), so that full-size checks can take experts one at a time.  Returns
    (grad_x_perm rows of the segment [count, H], grad_w_gate_up[ex] [2I, H],
    grad_w_down[ex] [H, I]); bf16 bits rounded once, or the float64 values."""
    e, two_i, h = w_gate_up.shape
    inter = two_i // 2
    f64 = lambda a: a if a.dtype == np.float64 else _bf16_f64(a)  # float64 inputs are taken as they are
    o, n = int(lay["expert_offsets"][ex]), int(lay["tokens_per_expert"][ex])
    x, dy = f64(x_perm[o:o + n]), f64(grad_y[o:o + n])
    wg, wu, wd = f64(w_gate_up[ex, :inter]), f64(w_gate_up[ex, inter:]), f64(w_down[ex])
    g = x @ wg.T
    u = x @ wu.T
    s = 1.0 / (1.0 + np.exp(-g))
    a = g * s * u
    da = dy @ wd
    dg = da * u * s * (1.0 + g * (1.0 - s))
    du = da * g * s
    gx = dg @ wg + du @ wu
    dwd = dy.T @ a
    dwgu = np.concatenate([dg.T @ x, du.T @ x])
    if not round_out:
        return gx, dwgu, dwd
    return bf16_round_array(gx), bf16_round_array(dwgu), bf16_round_array(dwd)


def expert_ffn_bwd_entries(x_perm, grad_y, lay, w_gate_up, w_down, rows=(), dwd=(), dwgu=()):
    """Selected outputs of expert_ffn_bwd, each from the same formulas taken over
    only the rows and columns it depends on (for shapes where the whole backward
    takes too long on the host): rows `rows` of grad_x_perm (rows inside the
    segments), entries (e, h, i) of grad_w_down and entries (e, j, h) of
    grad_w_gate_up (j < I: gate, j >= I: up).  fp64; each value rounded once to
    bf16.  Returns (grad_x rows [len(rows), H], dwd values, dwgu values) as bf16 bits.
    """
    e, two_i, h = w_gate_up.shape
    inter = two_i // 2
    offs = [int(v) for v in lay["expert_offsets"][:e]]
    cnts = [int(v) for v in lay["tokens_per_expert"][:e]]

    def expert_of(r):
        for ex in range(e):
            if offs[ex] <= r < offs[ex] + cnts[ex]:
                return ex
        raise ValueError(f"row {r} is outside every expert segment")

    gx = np.zeros((len(rows), h))
    for n, r in enumerate(rows):
        ex = expert_of(int(r))
        x, dy = _bf16_f64(x_perm[r]), _bf16_f64(grad_y[r])
        wg, wu, wd = _bf16_f64(w_gate_up[ex, :inter]), _bf16_f64(w_gate_up[ex, inter:]), _bf16_f64(w_down[ex])
        g, u = wg @ x, wu @ x
        sg = 1.0 / (1.0 + np.exp(-g))
        da = dy @ wd
        gx[n] = (da * u * sg * (1.0 + g * (1.0 - sg))) @ wg + (da * g * sg) @ wu

    segs = {}                          # expert -> its rows of x_perm and grad_y in fp64

    def columns(ex, i):
        """Per row of expert ex's segment: x, dy, g, u, sigmoid(g), dA of intermediate feature i."""
        if ex not in segs:
            o, n = offs[ex], cnts[ex]
            segs[ex] = (_bf16_f64(x_perm[o:o + n]), _bf16_f64(grad_y[o:o + n]))
        x, dy = segs[ex]
        g = x @ _bf16_f64(w_gate_up[ex, i])
        u = x @ _bf16_f64(w_gate_up[ex, inter + i])
        da = dy @ _bf16_f64(w_down[ex, :, i])
        return x, dy, g, u, 1.0 / (1.0 + np.exp(-g)), da

    vd = np.zeros(len(dwd))
    for n, (ex, hh, i) in enumerate(dwd):
        if cnts[ex] == 0:
            continue
        _, dy, g, u, sg, _ = columns(ex, i)
        vd[n] = dy[:, hh] @ (g * sg * u)
    vgu = np.zeros(len(dwgu))
    for n, (ex, j, hh) in enumerate(dwgu):
        if cnts[ex] == 0:
            continue
        x, _, g, u, sg, da = columns(ex, j % inter)
        col = da * u * sg * (1.0 + g * (1.0 - sg)) if j < inter else da * g * sg
        vgu[n] = col @ x[:, hh]
    return bf16_round_array(gx), bf16_round_array(vd), bf16_round_array(vgu)


def bf16_round(x: float) -> int:
    return int(lib().oracle_bf16_round(float(x)))
