"""MI355X (gfx950) single-GPU Mixture-of-Experts path: route -> dispatch ->
grouped SwiGLU expert FFN -> combine (+ the backward of combine, expert FFN and
dispatch).

A thin ctypes binding over the C ABI of libmoe_mi355x.so (include/moe.h).  It
only marshals arguments: tensors are passed as device pointers with
torch.cuda.current_stream() as the HIP stream, outputs and workspaces are
allocated with torch.  Every step of the path runs in the library's HIP
kernels; there is no other implementation behind these functions, and
importing this package fails if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libmoe_mi355x.so"

MOE_DT_F32 = 0
MOE_DT_BF16 = 1
MOE_DROP_POSITION, MOE_DROP_PROBS = 0, 1
(MOE_OP_ROUTE, MOE_OP_DISPATCH, MOE_OP_EXPERT_FFN, MOE_OP_COMBINE, MOE_OP_COMBINE_BWD, MOE_OP_EXPERT_FFN_BWD,
 MOE_OP_REROUTE, MOE_OP_EXPERT_FFN_MXFP8) = range(8)

# Every symbol include/moe.h declares.
EXPORTS = ("moe_layout_rows", "moe_workspace_size", "moe_route", "moe_route_random", "moe_dispatch",
           "moe_dispatch_noalloc", "moe_build_layout",
           "moe_dispatch_mxfp8", "moe_expert_ffn",
           "moe_expert_ffn_bwd", "moe_combine", "moe_dispatch_bwd", "moe_combine_bwd", "moe_status_string",
           "moe_version", "moe_replica_plan", "moe_reroute", "moe_replica_sync", "moe_replica_grad_reduce",
           "moe_expert_ffn_replicas", "moe_expert_ffn_bwd_replicas", "moe_mx_quantize", "moe_expert_ffn_mxfp8")


class MoeShape(C.Structure):
    _fields_ = [("n_tokens", C.c_int64), ("hidden", C.c_int64), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("capacity", C.c_int32), ("inter", C.c_int32), ("max_rows", C.c_int64), ("act_dtype", C.c_int32),
                ("row_align", C.c_int32), ("drop_policy", C.c_int32), ("reserved", C.c_int32)]


class MoeLayoutC(C.Structure):
    _fields_ = [(name, C.c_void_p) for name in ("tokens_per_expert", "expert_offsets", "ordinal", "assign_row",
                                                "row_src", "drop_mask", "pad_mask", "counters")]


class MoeError(RuntimeError):
    pass


def _load():
    if not _LIB_PATH.exists():
        raise ImportError(f"{_LIB_PATH} is missing: build it first (python __graft_entry__.py build, or "
                          f"python -m combine_router_softmax_amd._build)")
    lib = C.CDLL(str(_LIB_PATH))
    p, i32 = C.c_void_p, C.c_int
    sp = C.POINTER(MoeShape)
    lp = C.POINTER(MoeLayoutC)
    lib.moe_layout_rows.argtypes = [sp]
    lib.moe_layout_rows.restype = C.c_int64
    lib.moe_workspace_size.argtypes = [i32, sp, C.POINTER(C.c_size_t)]
    lib.moe_route.argtypes = [sp, p, p, p, p, p, p, p, p]
    lib.moe_route_random.argtypes = [sp, C.c_uint64, p, p, p, p, p, p, p]
    lib.moe_dispatch.argtypes = [sp, p, p, p, lp, p, p, p, C.c_size_t, p]
    lib.moe_dispatch_noalloc.argtypes = [sp, p, p, p, lp, p, p, p]
    lib.moe_build_layout.argtypes = [sp, p, p, lp, p, p, C.c_size_t, p]
    lib.moe_dispatch_mxfp8.argtypes = [sp, p, p, p, lp, p, p, p, p, C.c_size_t, p]
    lib.moe_expert_ffn.argtypes = [sp, p, lp, p, p, p, p, p, C.c_size_t, p]
    lib.moe_expert_ffn_bwd.argtypes = [sp, p, p, p, lp, p, p, p, p, p, p, C.c_size_t, p]
    lib.moe_combine.argtypes = [sp, p, p, lp, p, p]
    lib.moe_combine_bwd.argtypes = [sp, p, p, p, lp, p, p, p]
    lib.moe_dispatch_bwd.argtypes = [sp, p, lp, p, p]
    lib.moe_replica_plan.argtypes = [sp, p, i32, p, p]
    lib.moe_mx_quantize.argtypes = [C.c_int64, C.c_int64, p, p, p, p]
    lib.moe_expert_ffn_mxfp8.argtypes = [sp, p, p, lp, p, p, p, p, p, p, C.c_size_t, p]
    lib.moe_reroute.argtypes = [sp, p, p, i32, p, p, C.c_size_t, p]
    lib.moe_replica_sync.argtypes = [sp, p, i32, p, p, p, p, p]
    lib.moe_replica_grad_reduce.argtypes = [sp, p, i32, p, p, p, p, p]
    lib.moe_expert_ffn_replicas.argtypes = [sp, i32, p, lp, p, p, p, p, p, p, p, C.c_size_t, p]
    lib.moe_expert_ffn_bwd_replicas.argtypes = [sp, i32, p, p, p, lp, p, p, p, p, p, p, p, p, p, p, C.c_size_t, p]
    for f in ("moe_workspace_size", "moe_route", "moe_route_random", "moe_dispatch", "moe_dispatch_noalloc", "moe_build_layout", "moe_dispatch_mxfp8", "moe_expert_ffn", "moe_expert_ffn_bwd", "moe_combine",
              "moe_combine_bwd", "moe_dispatch_bwd", "moe_replica_plan", "moe_reroute", "moe_replica_sync",
              "moe_replica_grad_reduce", "moe_expert_ffn_replicas", "moe_expert_ffn_bwd_replicas", "moe_mx_quantize",
              "moe_expert_ffn_mxfp8"):
        getattr(lib, f).restype = i32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = C.c_char_p
    return lib


lib = _load()
library_path = str(_LIB_PATH)


def _check(status: int, what: str):
    if status != 0:
        raise MoeError(f"{what}: {lib.moe_status_string(status).decode()} (status {status})")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _act_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_DT_F32
    if t.dtype == torch.bfloat16:
        return MOE_DT_BF16
    raise TypeError(f"activations must be float32 or bfloat16, got {t.dtype}")


def _torch_dtype(dt: int):
    return torch.float32 if dt == MOE_DT_F32 else torch.bfloat16


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def make_shape(n_tokens, hidden, n_experts, top_k, capacity=0, inter=0, max_rows=0, act_dtype=MOE_DT_BF16,
               row_align=0, drop_policy=MOE_DROP_POSITION):
    return MoeShape(int(n_tokens), int(hidden), int(n_experts), int(top_k), int(capacity), int(inter), int(max_rows),
                    int(act_dtype), int(row_align), int(drop_policy), 0)


def workspace_size(op: int, shape: MoeShape) -> int:
    out = C.c_size_t(0)
    _check(lib.moe_workspace_size(op, C.byref(shape), C.byref(out)), "moe_workspace_size")
    return int(out.value)


def alloc_workspace(op: int, shape: MoeShape, device) -> torch.Tensor | None:
    """A device workspace for `op` at `shape` (include/moe.h moe_workspace_size), with
    256 bytes of slack for the 256-byte alignment the calls take.  Zero-filled: the
    dispatch and reroute workspaces must start with a zero header, which every call
    leaves zero again, so one workspace serves any number of calls in stream order."""
    n = workspace_size(op, shape)
    if n == 0:
        return None
    return torch.zeros(n + 256, dtype=torch.uint8, device=device)


def _workspace(op, shape, device):
    ws = alloc_workspace(op, shape, device)
    return ws, (0 if ws is None else ws.numel() - 256)


def _ws_ptr(ws):
    if ws is None:
        return None
    base = ws.data_ptr()
    return C.c_void_p((base + 255) & ~255)


@dataclass
class RouteOut:
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    routing_map: torch.Tensor | None
    tokens_per_expert: torch.Tensor | None


@dataclass
class Layout:
    """The dispatch layout (the "handle" moe_dispatch writes and the later calls read)."""
    n_tokens: int
    top_k: int
    n_experts: int
    capacity: int
    rows: int
    tokens_per_expert: torch.Tensor
    expert_offsets: torch.Tensor
    ordinal: torch.Tensor
    assign_row: torch.Tensor
    row_src: torch.Tensor
    drop_mask: torch.Tensor
    pad_mask: torch.Tensor
    counters: torch.Tensor
    row_align: int = 0
    drop_policy: int = MOE_DROP_POSITION

    @staticmethod
    def empty(n_tokens, top_k, n_experts, capacity, rows, device, row_align=0,
              drop_policy=MOE_DROP_POSITION) -> "Layout":
        i32 = dict(dtype=torch.int32, device=device)
        u8 = dict(dtype=torch.uint8, device=device)
        a = n_tokens * top_k
        return Layout(n_tokens, top_k, n_experts, capacity, rows, torch.empty(n_experts, **i32),
                      torch.empty(n_experts + 1, **i32), torch.empty(a, **i32), torch.empty(a, **i32),
                      torch.empty(rows, **i32), torch.empty(a, **u8), torch.empty(rows, **u8), torch.empty(4, **i32),
                      row_align, drop_policy)

    def c(self) -> MoeLayoutC:
        return MoeLayoutC(*[t.data_ptr() for t in (self.tokens_per_expert, self.expert_offsets, self.ordinal,
                                                   self.assign_row, self.row_src, self.drop_mask, self.pad_mask,
                                                   self.counters)])

    def shape(self, hidden, act_dtype, inter=0) -> MoeShape:
        return make_shape(self.n_tokens, hidden, self.n_experts, self.top_k, self.capacity, inter,
                          0 if self.capacity > 0 else self.rows, act_dtype, self.row_align, self.drop_policy)


def moe_route(logits: torch.Tensor, top_k: int, *, expert_bias: torch.Tensor | None = None,
              token_mask: torch.Tensor | None = None, routing_map: bool = True, counts: bool = True,
              out: RouteOut | None = None) -> RouteOut:
    """Router softmax / top-k (include/moe.h moe_route).  logits fp32 [N, E] on the GPU;
    expert_bias (optional, fp32 [E]): selection-only bias;
    token_mask (optional, uint8 or bool [N]): nonzero marks a padding token, routed nowhere."""
    _contig(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise TypeError("logits must be a float32 [N, E] tensor")
    n, e = logits.shape
    if expert_bias is not None:
        _contig(expert_bias, "expert_bias")
        if expert_bias.dtype != torch.float32 or tuple(expert_bias.shape) != (e,):
            raise TypeError("expert_bias must be a float32 [E] tensor")
    if token_mask is not None:
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        _contig(token_mask, "token_mask")
        if token_mask.dtype != torch.uint8 or tuple(token_mask.shape) != (n,):
            raise TypeError("token_mask must be a uint8 or bool [N] tensor")
    dev = logits.device
    if out is None:
        out = RouteOut(torch.empty((n, top_k), dtype=torch.int32, device=dev),
                       torch.empty((n, top_k), dtype=torch.float32, device=dev),
                       torch.empty((n, e), dtype=torch.uint8, device=dev) if routing_map else None,
                       torch.empty(e, dtype=torch.int32, device=dev) if counts else None)
    shape = make_shape(n, 1, e, top_k, act_dtype=MOE_DT_F32)
    _check(lib.moe_route(C.byref(shape), _ptr(logits), _ptr(expert_bias), _ptr(token_mask), _ptr(out.topk_idx),
                         _ptr(out.topk_w), _ptr(out.routing_map), _ptr(out.tokens_per_expert), _stream(dev)),
           "moe_route")
    return out


def moe_route_random(n_tokens: int, n_experts: int, top_k: int, seed: int, *, device="cuda",
                     expert_bias: torch.Tensor | None = None, token_mask: torch.Tensor | None = None,
                     routing_map: bool = True, counts: bool = True, out: RouteOut | None = None) -> RouteOut:
    """Force-balanced router (include/moe.h moe_route_random): moe_route over uniform random
    logits drawn from `seed` on the device."""
    dev = torch.device(device)
    n, e = int(n_tokens), int(n_experts)
    if expert_bias is not None:
        _contig(expert_bias, "expert_bias")
        if expert_bias.dtype != torch.float32 or tuple(expert_bias.shape) != (e,):
            raise TypeError("expert_bias must be a float32 [E] tensor")
    if token_mask is not None:
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        _contig(token_mask, "token_mask")
        if token_mask.dtype != torch.uint8 or tuple(token_mask.shape) != (n,):
            raise TypeError("token_mask must be a uint8 or bool [N] tensor")
    if out is None:
        out = RouteOut(torch.empty((n, top_k), dtype=torch.int32, device=dev),
                       torch.empty((n, top_k), dtype=torch.float32, device=dev),
                       torch.empty((n, e), dtype=torch.uint8, device=dev) if routing_map else None,
                       torch.empty(e, dtype=torch.int32, device=dev) if counts else None)
    shape = make_shape(n, 1, e, top_k, act_dtype=MOE_DT_F32)
    _check(lib.moe_route_random(C.byref(shape), C.c_uint64(seed & (2 ** 64 - 1)), _ptr(expert_bias),
                                _ptr(token_mask), _ptr(out.topk_idx), _ptr(out.topk_w), _ptr(out.routing_map),
                                _ptr(out.tokens_per_expert), _stream(dev)), "moe_route_random")
    return out


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor | None, n_experts: int, *,
                 capacity: int = 0, max_rows: int = 0, row_align: int = 0, drop_policy: int = MOE_DROP_POSITION,
                 w_perm: bool = True, layout: Layout | None = None, x_perm: torch.Tensor | None = None,
                 w_perm_out: torch.Tensor | None = None, workspace=None):
    """Layout + row scatter (include/moe.h moe_dispatch) -> (x_perm, w_perm, layout).
    row_align: dropless segments rounded up to multiples of this many rows (0: none);
    drop_policy: which assignments an over-full expert keeps with a capacity."""
    _contig(x, "x")
    _contig(topk_idx, "topk_idx")
    n, h = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    dt = _act_dtype(x)
    shape = make_shape(n, h, n_experts, k, capacity, 0, max_rows, dt, row_align, drop_policy)
    rows = int(lib.moe_layout_rows(C.byref(shape)))
    if rows < 0:
        _check(-1, "moe_dispatch")
    if layout is None:
        layout = Layout.empty(n, k, n_experts, capacity, rows, dev, row_align, drop_policy)
    if x_perm is None:
        x_perm = torch.empty((rows, h), dtype=x.dtype, device=dev)
    if w_perm and w_perm_out is None:
        w_perm_out = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_DISPATCH, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    _check(lib.moe_dispatch(C.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_w), C.byref(lc), _ptr(x_perm),
                            _ptr(w_perm_out if w_perm else None), _ws_ptr(ws), nbytes, _stream(dev)), "moe_dispatch")
    return x_perm, (w_perm_out if w_perm else None), layout


def moe_build_layout(topk_idx: torch.Tensor, topk_w: torch.Tensor | None, n_experts: int, *, hidden: int = 8,
                     act_dtype: int = MOE_DT_BF16, capacity: int = 0, max_rows: int = 0, row_align: int = 0,
                     drop_policy: int = MOE_DROP_POSITION, w_perm: bool = True, layout: Layout | None = None,
                     w_perm_out: torch.Tensor | None = None, workspace=None):
    """The dispatch layout without the row copy (include/moe.h moe_build_layout) -> (w_perm, layout).
    hidden / act_dtype only enter the shape checks (no activations are read)."""
    _contig(topk_idx, "topk_idx")
    n, k = topk_idx.shape
    dev = topk_idx.device
    shape = make_shape(n, hidden, n_experts, k, capacity, 0, max_rows, act_dtype, row_align, drop_policy)
    rows = int(lib.moe_layout_rows(C.byref(shape)))
    if rows < 0:
        _check(-1, "moe_build_layout")
    if layout is None:
        layout = Layout.empty(n, k, n_experts, capacity, rows, dev, row_align, drop_policy)
    if w_perm and w_perm_out is None:
        w_perm_out = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_DISPATCH, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    _check(lib.moe_build_layout(C.byref(shape), _ptr(topk_idx), _ptr(topk_w), C.byref(lc),
                                _ptr(w_perm_out if w_perm else None), _ws_ptr(ws), nbytes, _stream(dev)),
           "moe_build_layout")
    return (w_perm_out if w_perm else None), layout


def moe_dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor | None, n_experts: int, *,
                         capacity: int = 0, max_rows: int = 0, row_align: int = 0,
                         drop_policy: int = MOE_DROP_POSITION, w_perm: bool = True, layout: Layout | None = None,
                         x_perm: torch.Tensor | None = None, w_perm_out: torch.Tensor | None = None):
    """moe_dispatch on the library's static scratch (include/moe.h moe_dispatch_noalloc):
    no workspace.  The C entry point allocates nothing; pass layout, x_perm and
    w_perm_out to keep this call free of allocations on the Python side too."""
    _contig(x, "x")
    _contig(topk_idx, "topk_idx")
    n, h = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    shape = make_shape(n, h, n_experts, k, capacity, 0, max_rows, _act_dtype(x), row_align, drop_policy)
    rows = int(lib.moe_layout_rows(C.byref(shape)))
    if rows < 0:
        _check(-1, "moe_dispatch_noalloc")
    if layout is None:
        layout = Layout.empty(n, k, n_experts, capacity, rows, dev, row_align, drop_policy)
    if x_perm is None:
        x_perm = torch.empty((rows, h), dtype=x.dtype, device=dev)
    if w_perm and w_perm_out is None:
        w_perm_out = torch.empty(rows, dtype=torch.float32, device=dev)
    lc = layout.c()
    _check(lib.moe_dispatch_noalloc(C.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_w), C.byref(lc),
                                    _ptr(x_perm), _ptr(w_perm_out if w_perm else None), _stream(dev)),
           "moe_dispatch_noalloc")
    return x_perm, (w_perm_out if w_perm else None), layout


def moe_dispatch_mxfp8(x: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor | None, n_experts: int, *,
                       capacity: int = 0, max_rows: int = 0, row_align: int = 0,
                       drop_policy: int = MOE_DROP_POSITION, w_perm: bool = True, layout: Layout | None = None,
                       x_perm_q: torch.Tensor | None = None, x_perm_scale: torch.Tensor | None = None,
                       w_perm_out: torch.Tensor | None = None, workspace=None):
    """Layout + row scatter with MXFP8 quantisation (include/moe.h moe_dispatch_mxfp8):
    bf16 x [N, H], H % 32 == 0 -> (x_perm_q uint8 [R, H] E4M3 codes, x_perm_scale uint8
    [R, H/32] E8M0 codes, w_perm, layout).  Options as moe_dispatch."""
    _contig(x, "x")
    _contig(topk_idx, "topk_idx")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    n, h = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    shape = make_shape(n, h, n_experts, k, capacity, 0, max_rows, MOE_DT_BF16, row_align, drop_policy)
    rows = int(lib.moe_layout_rows(C.byref(shape)))
    if rows < 0:
        _check(-1, "moe_dispatch_mxfp8")
    if layout is None:
        layout = Layout.empty(n, k, n_experts, capacity, rows, dev, row_align, drop_policy)
    if x_perm_q is None:
        x_perm_q = torch.empty((rows, h), dtype=torch.uint8, device=dev)
    if x_perm_scale is None:
        x_perm_scale = torch.empty((rows, h // 32), dtype=torch.uint8, device=dev)
    for t, name in ((x_perm_q, "x_perm_q"), (x_perm_scale, "x_perm_scale")):
        _contig(t, name)
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must be uint8")
    if w_perm and w_perm_out is None:
        w_perm_out = torch.empty(rows, dtype=torch.float32, device=dev)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_DISPATCH, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    _check(lib.moe_dispatch_mxfp8(C.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_w), C.byref(lc),
                                  _ptr(x_perm_q), _ptr(x_perm_scale), _ptr(w_perm_out if w_perm else None),
                                  _ws_ptr(ws), nbytes, _stream(dev)), "moe_dispatch_mxfp8")
    return x_perm_q, x_perm_scale, (w_perm_out if w_perm else None), layout


def _bf16(*named):
    for t, name in named:
        _contig(t, name)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")


def _ffn_shapes(x_perm, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica):
    """(rows, H, I, R) of a grouped FFN call; the masters and the R replica slots
    together are the layout's experts."""
    _bf16((x_perm, "x_perm"), (w_gate_up, "w_gate_up"), (w_down, "w_down"))
    rows, h = x_perm.shape
    e, two_i, h2 = w_gate_up.shape
    inter = two_i // 2
    r = 0
    if w_gate_up_replica is not None or w_down_replica is not None:
        _bf16((w_gate_up_replica, "w_gate_up_replica"), (w_down_replica, "w_down_replica"))
        r = w_gate_up_replica.shape[0]
        if (tuple(w_gate_up_replica.shape) != (r, two_i, h) or tuple(w_down_replica.shape) != (r, h, inter)):
            raise ValueError("replica weights must be [R, 2I, H] and [R, H, I]")
    if h2 != h or tuple(w_down.shape) != (e, h, inter) or e + r != layout.n_experts or rows != layout.rows:
        raise ValueError("inconsistent expert FFN shapes")
    return rows, h, inter, r


def _expert_ffn(x_perm, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica, y, gate_up, save_gate_up,
                workspace):
    rows, h, inter, r = _ffn_shapes(x_perm, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica)
    dev = x_perm.device
    shape = layout.shape(h, MOE_DT_BF16, inter)
    if y is None:
        y = torch.empty_like(x_perm)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_EXPERT_FFN, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    if save_gate_up and gate_up is None:
        gate_up = torch.empty((rows, 2 * inter), dtype=torch.bfloat16, device=dev)
    if gate_up is not None:
        _contig(gate_up, "gate_up")
        if gate_up.dtype != torch.bfloat16 or tuple(gate_up.shape) != (rows, 2 * inter):
            raise ValueError("gate_up must be bfloat16 [R, 2I]")
    if r == 0 and w_gate_up_replica is None:
        _check(lib.moe_expert_ffn(C.byref(shape), _ptr(x_perm), C.byref(lc), _ptr(w_gate_up), _ptr(w_down), _ptr(y),
                                  _ptr(gate_up), _ws_ptr(ws), nbytes, _stream(dev)), "moe_expert_ffn")
    else:
        _check(lib.moe_expert_ffn_replicas(C.byref(shape), r, _ptr(x_perm), C.byref(lc), _ptr(w_gate_up),
                                           _ptr(w_down), _ptr(w_gate_up_replica), _ptr(w_down_replica), _ptr(y),
                                           _ptr(gate_up), _ws_ptr(ws), nbytes, _stream(dev)),
               "moe_expert_ffn_replicas")
    return (y, gate_up) if gate_up is not None else y


def moe_expert_ffn(x_perm: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor, w_down: torch.Tensor, *,
                   y: torch.Tensor | None = None, gate_up: torch.Tensor | None = None, save_gate_up: bool = False,
                   workspace=None):
    """Grouped SwiGLU FFN (include/moe.h moe_expert_ffn): bf16 x_perm [R, H], w_gate_up [E, 2I, H], w_down [E, H, I].
    Returns y [R, H]; with save_gate_up (or a gate_up buffer [R, 2I]) returns (y, gate_up), the
    pre-activations moe_expert_ffn_bwd can take."""
    return _expert_ffn(x_perm, layout, w_gate_up, w_down, None, None, y, gate_up, save_gate_up, workspace)


def moe_expert_ffn_replicas(x_perm: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor, w_down: torch.Tensor,
                            w_gate_up_replica: torch.Tensor, w_down_replica: torch.Tensor, *,
                            y: torch.Tensor | None = None, gate_up: torch.Tensor | None = None,
                            save_gate_up: bool = False, workspace=None):
    """moe_expert_ffn over physical experts (include/moe.h moe_expert_ffn_replicas): the layout's
    last R experts are replica slots with weights w_gate_up_replica [R, 2I, H], w_down_replica [R, H, I]."""
    return _expert_ffn(x_perm, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica, y, gate_up,
                       save_gate_up, workspace)


def _expert_ffn_bwd(x_perm, grad_y, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica, gate_up,
                    grad_x_perm, grad_w_gate_up, grad_w_down, grad_w_gate_up_replica, grad_w_down_replica,
                    workspace):
    rows, h, inter, r = _ffn_shapes(x_perm, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica)
    _bf16((grad_y, "grad_y"))
    if tuple(grad_y.shape) != (rows, h):
        raise ValueError("inconsistent expert FFN shapes")
    if gate_up is not None:
        _contig(gate_up, "gate_up")
        if gate_up.dtype != torch.bfloat16 or tuple(gate_up.shape) != (rows, 2 * inter):
            raise ValueError("gate_up must be bfloat16 [R, 2I]")
    dev = x_perm.device
    shape = layout.shape(h, MOE_DT_BF16, inter)
    if grad_x_perm is None:
        grad_x_perm = torch.empty_like(x_perm)
    if grad_w_gate_up is None:
        grad_w_gate_up = torch.empty_like(w_gate_up)
    if grad_w_down is None:
        grad_w_down = torch.empty_like(w_down)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_EXPERT_FFN_BWD, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    if w_gate_up_replica is None:
        _check(lib.moe_expert_ffn_bwd(C.byref(shape), _ptr(x_perm), _ptr(grad_y), _ptr(gate_up), C.byref(lc),
                                      _ptr(w_gate_up), _ptr(w_down), _ptr(grad_x_perm), _ptr(grad_w_gate_up),
                                      _ptr(grad_w_down), _ws_ptr(ws), nbytes, _stream(dev)), "moe_expert_ffn_bwd")
        return grad_x_perm, grad_w_gate_up, grad_w_down
    if grad_w_gate_up_replica is None:
        grad_w_gate_up_replica = torch.empty_like(w_gate_up_replica)
    if grad_w_down_replica is None:
        grad_w_down_replica = torch.empty_like(w_down_replica)
    _check(lib.moe_expert_ffn_bwd_replicas(C.byref(shape), r, _ptr(x_perm), _ptr(grad_y), _ptr(gate_up), C.byref(lc),
                                           _ptr(w_gate_up), _ptr(w_down), _ptr(w_gate_up_replica),
                                           _ptr(w_down_replica), _ptr(grad_x_perm), _ptr(grad_w_gate_up),
                                           _ptr(grad_w_down), _ptr(grad_w_gate_up_replica),
                                           _ptr(grad_w_down_replica), _ws_ptr(ws), nbytes, _stream(dev)),
           "moe_expert_ffn_bwd_replicas")
    return grad_x_perm, grad_w_gate_up, grad_w_down, grad_w_gate_up_replica, grad_w_down_replica


def moe_expert_ffn_bwd(x_perm: torch.Tensor, grad_y: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor,
                       w_down: torch.Tensor, *, gate_up: torch.Tensor | None = None,
                       grad_x_perm: torch.Tensor | None = None, grad_w_gate_up: torch.Tensor | None = None,
                       grad_w_down: torch.Tensor | None = None, workspace=None):
    """Backward of the grouped SwiGLU FFN (include/moe.h moe_expert_ffn_bwd)
    -> (grad_x_perm [R, H], grad_w_gate_up [E, 2I, H], grad_w_down [E, H, I]), all bf16.
    gate_up: the pre-activations saved by moe_expert_ffn (None: recomputed)."""
    return _expert_ffn_bwd(x_perm, grad_y, layout, w_gate_up, w_down, None, None, gate_up, grad_x_perm,
                           grad_w_gate_up, grad_w_down, None, None, workspace)


def moe_expert_ffn_bwd_replicas(x_perm: torch.Tensor, grad_y: torch.Tensor, layout: Layout, w_gate_up: torch.Tensor,
                                w_down: torch.Tensor, w_gate_up_replica: torch.Tensor, w_down_replica: torch.Tensor,
                                *, gate_up: torch.Tensor | None = None, grad_x_perm: torch.Tensor | None = None,
                                grad_w_gate_up: torch.Tensor | None = None, grad_w_down: torch.Tensor | None = None,
                                grad_w_gate_up_replica: torch.Tensor | None = None,
                                grad_w_down_replica: torch.Tensor | None = None, workspace=None):
    """Backward with replica slots (include/moe.h moe_expert_ffn_bwd_replicas) -> (grad_x_perm,
    grad_w_gate_up, grad_w_down, grad_w_gate_up_replica, grad_w_down_replica)."""
    return _expert_ffn_bwd(x_perm, grad_y, layout, w_gate_up, w_down, w_gate_up_replica, w_down_replica, gate_up,
                           grad_x_perm, grad_w_gate_up, grad_w_down, grad_w_gate_up_replica, grad_w_down_replica,
                           workspace)


def moe_mx_quantize(x: torch.Tensor, *, q: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """MXFP8 of a bf16 matrix along its rows (include/moe.h moe_mx_quantize): x [..., cols]
    -> (q uint8 [..., cols] E4M3 codes, scale uint8 [..., cols/32] E8M0 codes)."""
    _bf16((x, "x"))
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=x.device)
    _check(lib.moe_mx_quantize(rows, cols, _ptr(x), _ptr(q), _ptr(scale), _stream(x.device)), "moe_mx_quantize")
    return q, scale


def moe_expert_ffn_mxfp8(x_perm_q: torch.Tensor, x_perm_scale: torch.Tensor, layout: Layout,
                         w_gate_up_q: torch.Tensor, w_gate_up_scale: torch.Tensor, w_down_q: torch.Tensor,
                         w_down_scale: torch.Tensor, *, y: torch.Tensor | None = None, workspace=None):
    """Grouped SwiGLU FFN over MXFP8 operands (include/moe.h moe_expert_ffn_mxfp8): x_perm_q [R, H] +
    x_perm_scale [R, H/32] (moe_dispatch_mxfp8), weights from moe_mx_quantize: w_gate_up_q
    [E, 2I, H] + [E, 2I, H/32], w_down_q [E, H, I] + [E, H, I/32] -> y bf16 [R, H]."""
    for t, name in ((x_perm_q, "x_perm_q"), (x_perm_scale, "x_perm_scale"), (w_gate_up_q, "w_gate_up_q"),
                    (w_gate_up_scale, "w_gate_up_scale"), (w_down_q, "w_down_q"), (w_down_scale, "w_down_scale")):
        _contig(t, name)
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must be uint8")
    rows, h = x_perm_q.shape
    e, two_i, h2 = w_gate_up_q.shape
    inter = two_i // 2
    if (h2 != h or tuple(w_down_q.shape) != (e, h, inter) or tuple(x_perm_scale.shape) != (rows, h // 32)
            or tuple(w_gate_up_scale.shape) != (e, two_i, h // 32) or tuple(w_down_scale.shape) != (e, h, inter // 32)
            or e != layout.n_experts or rows != layout.rows):
        raise ValueError("inconsistent MXFP8 expert FFN shapes")
    dev = x_perm_q.device
    shape = layout.shape(h, MOE_DT_BF16, inter)
    if y is None:
        y = torch.empty((rows, h), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_EXPERT_FFN_MXFP8, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    lc = layout.c()
    _check(lib.moe_expert_ffn_mxfp8(C.byref(shape), _ptr(x_perm_q), _ptr(x_perm_scale), C.byref(lc), _ptr(w_gate_up_q),
                                    _ptr(w_gate_up_scale), _ptr(w_down_q), _ptr(w_down_scale), _ptr(y), _ws_ptr(ws),
                                    nbytes, _stream(dev)), "moe_expert_ffn_mxfp8")
    return y


def moe_replica_plan(tokens_per_expert: torch.Tensor, n_replicas: int, *, out: torch.Tensor | None = None):
    """Hot-expert placement (include/moe.h moe_replica_plan) -> replica_of int32 [n_replicas]."""
    _contig(tokens_per_expert, "tokens_per_expert")
    e = tokens_per_expert.numel()
    dev = tokens_per_expert.device
    if out is None:
        out = torch.empty(n_replicas, dtype=torch.int32, device=dev)
    shape = make_shape(0, 1, e, 1)
    _check(lib.moe_replica_plan(C.byref(shape), _ptr(tokens_per_expert), n_replicas, _ptr(out), _stream(dev)),
           "moe_replica_plan")
    return out


def moe_reroute(topk_idx: torch.Tensor, n_experts: int, replica_of: torch.Tensor, *, out: torch.Tensor | None = None,
                workspace=None):
    """Logical -> physical expert ids (include/moe.h moe_reroute) -> phys_idx int32 [N, k]."""
    _contig(topk_idx, "topk_idx")
    _contig(replica_of, "replica_of")
    n, k = topk_idx.shape
    dev = topk_idx.device
    if out is None:
        out = torch.empty_like(topk_idx)
    shape = make_shape(n, 1, n_experts, k)
    if workspace is None:
        ws, nbytes = _workspace(MOE_OP_REROUTE, shape, dev)
    else:
        ws, nbytes = workspace, workspace.numel() - 256
    _check(lib.moe_reroute(C.byref(shape), _ptr(topk_idx), _ptr(replica_of), replica_of.numel(), _ptr(out),
                           _ws_ptr(ws), nbytes, _stream(dev)), "moe_reroute")
    return out


def moe_replica_sync(w_gate_up: torch.Tensor, w_down: torch.Tensor, replica_of: torch.Tensor, *,
                     w_gate_up_replica: torch.Tensor | None = None, w_down_replica: torch.Tensor | None = None):
    """Replica weight sync (include/moe.h moe_replica_sync) -> (w_gate_up_replica [R, 2I, H],
    w_down_replica [R, H, I])."""
    _bf16((w_gate_up, "w_gate_up"), (w_down, "w_down"))
    _contig(replica_of, "replica_of")
    e, two_i, h = w_gate_up.shape
    r = replica_of.numel()
    if w_gate_up_replica is None:
        w_gate_up_replica = torch.empty((r, two_i, h), dtype=torch.bfloat16, device=w_gate_up.device)
    if w_down_replica is None:
        w_down_replica = torch.empty((r, h, two_i // 2), dtype=torch.bfloat16, device=w_gate_up.device)
    shape = make_shape(0, h, e, 1, inter=two_i // 2)
    _check(lib.moe_replica_sync(C.byref(shape), _ptr(replica_of), r, _ptr(w_gate_up), _ptr(w_down),
                                _ptr(w_gate_up_replica), _ptr(w_down_replica), _stream(w_gate_up.device)),
           "moe_replica_sync")
    return w_gate_up_replica, w_down_replica


def moe_replica_grad_reduce(grad_w_gate_up: torch.Tensor, grad_w_down: torch.Tensor,
                            grad_w_gate_up_replica: torch.Tensor, grad_w_down_replica: torch.Tensor,
                            replica_of: torch.Tensor):
    """Adds the replica slots' weight gradients into their masters' (include/moe.h
    moe_replica_grad_reduce), in place -> (grad_w_gate_up, grad_w_down)."""
    _bf16((grad_w_gate_up, "grad_w_gate_up"), (grad_w_down, "grad_w_down"),
          (grad_w_gate_up_replica, "grad_w_gate_up_replica"), (grad_w_down_replica, "grad_w_down_replica"))
    _contig(replica_of, "replica_of")
    e, two_i, h = grad_w_gate_up.shape
    shape = make_shape(0, h, e, 1, inter=two_i // 2)
    _check(lib.moe_replica_grad_reduce(C.byref(shape), _ptr(replica_of), replica_of.numel(),
                                       _ptr(grad_w_gate_up_replica), _ptr(grad_w_down_replica), _ptr(grad_w_gate_up),
                                       _ptr(grad_w_down), _stream(grad_w_gate_up.device)), "moe_replica_grad_reduce")
    return grad_w_gate_up, grad_w_down


def moe_combine(y: torch.Tensor, topk_w: torch.Tensor, layout: Layout, *, out: torch.Tensor | None = None):
    """Probability-weighted combine (include/moe.h moe_combine) -> out [N, H]."""
    _contig(y, "y")
    _contig(topk_w, "topk_w")
    h = y.shape[1]
    dt = _act_dtype(y)
    if out is None:
        out = torch.empty((layout.n_tokens, h), dtype=y.dtype, device=y.device)
    shape = layout.shape(h, dt)
    lc = layout.c()
    _check(lib.moe_combine(C.byref(shape), _ptr(y), _ptr(topk_w), C.byref(lc), _ptr(out), _stream(y.device)),
           "moe_combine")
    return out


def moe_dispatch_bwd(grad_x_perm: torch.Tensor, layout: Layout, *, out: torch.Tensor | None = None):
    """Backward of the row scatter of moe_dispatch (include/moe.h moe_dispatch_bwd) -> grad_x [N, H]."""
    _contig(grad_x_perm, "grad_x_perm")
    h = grad_x_perm.shape[1]
    dt = _act_dtype(grad_x_perm)
    if out is None:
        out = torch.empty((layout.n_tokens, h), dtype=grad_x_perm.dtype, device=grad_x_perm.device)
    shape = layout.shape(h, dt)
    lc = layout.c()
    _check(lib.moe_dispatch_bwd(C.byref(shape), _ptr(grad_x_perm), C.byref(lc), _ptr(out),
                                _stream(grad_x_perm.device)), "moe_dispatch_bwd")
    return out


def moe_combine_bwd(grad_out: torch.Tensor, y: torch.Tensor, topk_w: torch.Tensor, layout: Layout, *,
                    grad_y: torch.Tensor | None = None, grad_w: torch.Tensor | None = None):
    """Backward of moe_combine (include/moe.h moe_combine_bwd) -> (grad_y [R, H], grad_w fp32 [N, k])."""
    _contig(grad_out, "grad_out")
    _contig(y, "y")
    h = y.shape[1]
    dt = _act_dtype(y)
    if grad_out.dtype != y.dtype:
        raise TypeError("grad_out and y must have the same dtype")
    if grad_y is None:
        grad_y = torch.empty_like(y)
    if grad_w is None:
        grad_w = torch.empty((layout.n_tokens, layout.top_k), dtype=torch.float32, device=y.device)
    shape = layout.shape(h, dt)
    lc = layout.c()
    _check(lib.moe_combine_bwd(C.byref(shape), _ptr(grad_out), _ptr(y), _ptr(topk_w), C.byref(lc), _ptr(grad_y),
                               _ptr(grad_w), _stream(y.device)), "moe_combine_bwd")
    return grad_y, grad_w


__all__ = ["moe_route", "moe_route_random", "moe_dispatch", "moe_dispatch_mxfp8", "moe_mx_quantize",
           "moe_expert_ffn_mxfp8", "moe_replica_plan", "moe_reroute",
           "moe_replica_sync", "moe_replica_grad_reduce", "moe_expert_ffn_replicas", "moe_expert_ffn_bwd_replicas", "moe_expert_ffn", "moe_expert_ffn_bwd", "moe_combine", "moe_combine_bwd",
           "moe_dispatch_bwd",
           "Layout", "RouteOut",
           "MoeError", "make_shape", "workspace_size", "lib", "library_path", "EXPORTS"]
