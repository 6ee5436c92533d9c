"""Host-side checks of the C ABI library (no GPU needed, no kernel launched):
the library loads, exports every function include/moe.h declares, sizes its
workspaces, and rejects bad arguments before touching the device."""
from __future__ import annotations

import ctypes as C
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


def header_functions():
    text = (ROOT / "include" / "moe.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def moe():
    import combine_router_softmax_amd as m
    return m


def test_library_exports_every_declared_function(moe):
    declared = header_functions()
    assert len(declared) == 23, declared
    assert sorted(moe.EXPORTS) == declared
    for name in declared:
        assert hasattr(moe.lib, name), name
    assert moe.lib.moe_version().decode().count(".") == 2


def test_library_is_built_for_gfx950(moe):
    data = Path(moe.library_path).read_bytes()
    assert b"gfx950" in data


def test_status_strings(moe):
    for st in range(0, -6, -1):
        s = moe.lib.moe_status_string(st).decode()
        assert s and s != "unknown status"
    assert moe.lib.moe_status_string(-99).decode() == "unknown status"


def test_layout_rows_and_workspace_sizes(moe):
    s = moe.make_shape(4096, 7168, 256, 8)
    assert moe.lib.moe_layout_rows(C.byref(s)) == 32768
    s = moe.make_shape(4096, 7168, 256, 8, capacity=160)
    assert moe.lib.moe_layout_rows(C.byref(s)) == 40960
    s = moe.make_shape(16384, 7168, 32, 8, max_rows=32768)
    assert moe.lib.moe_layout_rows(C.byref(s)) == 32768
    assert moe.workspace_size(moe.MOE_OP_ROUTE, s) == 0
    assert moe.workspace_size(moe.MOE_OP_COMBINE, s) == 0
    tiles = (16384 * 8 + 2047) // 2048
    # a 256-byte header, then one 64-bit status word per tile and bin (32 experts + invalid ids)
    assert moe.workspace_size(moe.MOE_OP_DISPATCH, s) >= 256 + tiles * 33 * 8
    s = moe.make_shape(8192, 4096, 128, 8, inter=1536)
    assert moe.workspace_size(moe.MOE_OP_EXPERT_FFN, s) >= 65536 * 1536 * 2
    assert moe.workspace_size(moe.MOE_OP_EXPERT_FFN_BWD, s) >= 65536 * 3 * 1536 * 2   # [R, 3I] bf16
    # no tokens: still the header and one tile (the scan writes the zero counts and offsets)
    assert moe.workspace_size(moe.MOE_OP_DISPATCH, moe.make_shape(0, 64, 4, 2)) >= 256 + 5 * 8
    # dropping by weight lists every assignment by expert: room for N*k ints more
    pos = moe.workspace_size(moe.MOE_OP_DISPATCH, moe.make_shape(4096, 7168, 256, 8, capacity=160))
    probs = moe.workspace_size(moe.MOE_OP_DISPATCH, moe.make_shape(4096, 7168, 256, 8, capacity=160,
                                                                  drop_policy=moe.MOE_DROP_PROBS))
    assert probs >= pos + 4096 * 8 * 4 + 257 * 4
    # aligned dropless segments: room for E * (A - 1) pad rows; a row budget or a capacity fixes R
    assert moe.lib.moe_layout_rows(C.byref(moe.make_shape(4096, 7168, 256, 8, row_align=64))) == 32768 + 256 * 63
    assert moe.lib.moe_layout_rows(C.byref(moe.make_shape(4096, 7168, 256, 8, row_align=1))) == 32768
    assert moe.lib.moe_layout_rows(C.byref(moe.make_shape(16384, 7168, 32, 8, max_rows=40000, row_align=16))) == 40000


@pytest.mark.parametrize("field,value,status", [
    ("n_tokens", -1, -1), ("hidden", 0, -1), ("n_experts", 0, -1), ("n_experts", 1025, -4), ("top_k", 0, -1),
    ("act_dtype", 7, -1), ("row_align", 3, -1), ("row_align", 2048, -1), ("row_align", -2, -1), ("max_rows", -5, -1),
    ("drop_policy", 2, -1), ("drop_policy", -1, -1), ("reserved", 1, -1),
])
def test_bad_shapes_are_rejected(moe, field, value, status):
    s = moe.make_shape(16, 64, 8, 2)
    setattr(s, field, value)
    out = C.c_size_t(0)
    assert moe.lib.moe_workspace_size(moe.MOE_OP_DISPATCH, C.byref(s), C.byref(out)) == status
    assert moe.lib.moe_layout_rows(C.byref(s)) == -1


def test_noalloc_dispatch_rejects_shapes_beyond_its_scratch(moe):
    """moe_dispatch_noalloc checks its scratch need on the host, before any HIP call."""
    s = moe.make_shape(5_000_000, 64, 256, 8)      # 40M assignments: far more status words than 8 MiB
    p = C.c_void_p(4096)
    lay = moe.MoeLayoutC(*([4096] * 8))
    need = moe.workspace_size(moe.MOE_OP_DISPATCH, s)
    assert need > 8 << 20
    assert moe.lib.moe_dispatch_noalloc(C.byref(s), p, p, p, C.byref(lay), p, None, None) == -3
    assert moe.lib.moe_dispatch_noalloc(None, p, p, p, C.byref(lay), p, None, None) == -1


def test_validation_errors_enqueue_nothing(moe):
    """Every call below fails host-side validation, so no HIP call is made."""
    lib = moe.lib
    p = C.c_void_p(4096)          # a fake, 16-byte-aligned "device" address: never dereferenced
    odd = C.c_void_p(4096 + 2)
    s = moe.make_shape(16, 64, 8, 9, act_dtype=moe.MOE_DT_F32)
    assert lib.moe_route(C.byref(s), p, None, None, p, p, None, None, None) == -1    # k > E
    s = moe.make_shape(16, 64, 8, 2, act_dtype=moe.MOE_DT_F32)
    assert lib.moe_route(C.byref(s), None, None, None, p, p, None, None, None) == -1  # null logits
    assert lib.moe_route(C.byref(s), odd, None, None, p, p, None, None, None) == -2   # misaligned
    assert lib.moe_route(C.byref(s), p, odd, None, p, p, None, None, None) == -2     # misaligned bias
    assert lib.moe_route(None, p, None, None, p, p, None, None, None) == -1
    lay = moe.MoeLayoutC(*([4096] * 8))
    s = moe.make_shape(16, 60, 8, 2, act_dtype=moe.MOE_DT_BF16)                # 120-byte rows
    assert lib.moe_dispatch(C.byref(s), p, p, p, C.byref(lay), p, p, p, 1 << 20, None) == -2
    s = moe.make_shape(16, 64, 8, 2, act_dtype=moe.MOE_DT_BF16)
    assert lib.moe_dispatch(C.byref(s), odd, p, p, C.byref(lay), p, p, p, 1 << 20, None) == -2
    assert lib.moe_dispatch(C.byref(s), p, p, p, C.byref(lay), p, p, p, 0, None) == -3       # no workspace
    assert lib.moe_dispatch(C.byref(s), p, p, p, C.byref(lay), p, p, odd, 1 << 20, None) == -3  # unaligned ws
    assert lib.moe_dispatch(C.byref(s), p, p, p, None, p, p, p, 1 << 20, None) == -1
    s = moe.make_shape(16, 64, 8, 2, capacity=4, drop_policy=moe.MOE_DROP_PROBS)  # the policy needs topk_w
    assert lib.moe_dispatch(C.byref(s), p, p, None, C.byref(lay), p, None, p, 1 << 20, None) == -1
    s = moe.make_shape(16, 64, 8, 2, capacity=6, row_align=4)                   # C not a multiple of A
    assert lib.moe_dispatch(C.byref(s), p, p, p, C.byref(lay), p, p, p, 1 << 20, None) == -4
    s = moe.make_shape(16, 64, 8, 2, capacity=4, max_rows=7)                   # max_rows != E*C
    assert lib.moe_dispatch(C.byref(s), p, p, p, C.byref(lay), p, p, p, 1 << 20, None) == -1
    mx = lib.moe_dispatch_mxfp8
    q8, s8 = C.c_void_p(8192), C.c_void_p(12288)
    s = moe.make_shape(16, 64, 8, 2, act_dtype=moe.MOE_DT_F32)                 # fp32 input
    assert mx(C.byref(s), p, p, p, C.byref(lay), q8, s8, p, p, 1 << 20, None) == -4
    s = moe.make_shape(16, 48, 8, 2)                                           # H % 32 != 0
    assert mx(C.byref(s), p, p, p, C.byref(lay), q8, s8, p, p, 1 << 20, None) == -4
    s = moe.make_shape(16, 64, 8, 2)
    assert mx(C.byref(s), p, p, p, C.byref(lay), C.c_void_p(8200), s8, p, p, 1 << 20, None) == -2  # q misaligned
    assert mx(C.byref(s), p, p, p, C.byref(lay), q8, None, p, p, 1 << 20, None) == -1   # no scale buffer
    assert mx(C.byref(s), p, p, p, C.byref(lay), q8, q8, p, p, 1 << 20, None) == -1     # scales alias codes
    assert mx(C.byref(s), odd, p, p, C.byref(lay), q8, s8, p, p, 1 << 20, None) == -2  # x misaligned
    assert mx(C.byref(s), p, p, p, C.byref(lay), q8, s8, p, p, 0, None) == -3          # no workspace
    assert mx(C.byref(s), p, p, p, None, q8, s8, p, p, 1 << 20, None) == -1
    # hot-expert replication
    s = moe.make_shape(16, 64, 8, 2, inter=64)
    rep, tpe = C.c_void_p(4096), C.c_void_p(8192)
    assert lib.moe_replica_plan(C.byref(s), tpe, 4, None, None) == -1           # no replica_of
    assert lib.moe_replica_plan(C.byref(s), None, 4, rep, None) == -1           # no counts
    assert lib.moe_replica_plan(C.byref(s), tpe, -1, rep, None) == -1
    assert lib.moe_replica_plan(C.byref(s), tpe, 1025, rep, None) == -4
    assert lib.moe_replica_plan(C.byref(s), C.c_void_p(8194), 4, rep, None) == -2
    assert lib.moe_reroute(C.byref(s), p, rep, 4, p, p, 0, None) == -3         # no workspace
    assert lib.moe_reroute(C.byref(s), p, rep, 1020, p, p, 1 << 20, None) == -4  # E + R > 1024
    assert lib.moe_reroute(C.byref(s), None, rep, 4, p, p, 1 << 20, None) == -1
    assert lib.moe_reroute(C.byref(s), odd, rep, 4, p, p, 1 << 20, None) == -2
    w1, w2, w3, w4 = (C.c_void_p(v) for v in (1 << 16, 1 << 17, 1 << 18, 1 << 19))
    assert lib.moe_replica_sync(C.byref(s), rep, 2, w1, w2, w3, w3, None) == -1   # replica buffers alias
    assert lib.moe_replica_sync(C.byref(s), rep, 2, w1, w2, w1, w4, None) == -1   # replica aliases a master
    assert lib.moe_replica_sync(C.byref(s), rep, 2, w1, w2, odd, w4, None) == -2
    assert lib.moe_replica_sync(C.byref(s), rep, 2, w1, None, w3, w4, None) == -1
    assert lib.moe_replica_sync(C.byref(s), rep, 0, None, None, None, None, None) == 0  # nothing to do
    assert lib.moe_replica_grad_reduce(C.byref(s), rep, 2, w3, w4, w1, w1, None) == -1  # masters alias
    assert lib.moe_replica_grad_reduce(C.byref(s), rep, 2, w3, w4, w3, w2, None) == -1  # master aliases a replica
    assert lib.moe_replica_grad_reduce(C.byref(s), None, 2, w3, w4, w1, w2, None) == -1
    s96 = moe.make_shape(16, 64, 8, 2, inter=96)
    assert lib.moe_replica_sync(C.byref(s96), rep, 2, w1, w2, w3, w4, None) == -4     # I % 64
    ffr = lib.moe_expert_ffn_replicas
    assert ffr(C.byref(s), 8, p, C.byref(lay), w1, w2, w3, w4, p, None, p, 1 << 30, None) == -1  # R >= P
    assert ffr(C.byref(s), 2, p, C.byref(lay), w1, w2, None, w4, p, None, p, 1 << 30, None) == -1
    assert ffr(C.byref(s), 2, p, C.byref(lay), w1, w2, odd, w4, p, None, p, 1 << 30, None) == -2
    assert ffr(C.byref(s), 2, p, C.byref(lay), w1, w2, w1, w4, p, None, p, 1 << 30, None) == -1  # aliases
    bwr = lib.moe_expert_ffn_bwd_replicas
    g1, g2 = C.c_void_p(1 << 20), C.c_void_p(1 << 21)
    q, r = C.c_void_p(8192), C.c_void_p(12288)
    assert bwr(C.byref(s), 2, p, p, None, C.byref(lay), w1, w2, w3, w4, q, r, C.c_void_p(16384), None, g2, p,
               1 << 30, None) == -1                                             # no replica grad buffer
    assert bwr(C.byref(s), 2, p, p, None, C.byref(lay), w1, w2, w3, w4, q, r, C.c_void_p(16384), g1, g1, p,
               1 << 30, None) == -1                                             # replica grads alias
    assert bwr(C.byref(s), 2, p, p, None, C.byref(lay), w1, w2, w3, w4, q, r, C.c_void_p(16384), g1, w4, p,
               1 << 30, None) == -1                                             # replica grad aliases a weight
    # MXFP8 quantisation and FFN
    assert lib.moe_mx_quantize(4, 48, p, q, r, None) == -4                  # cols % 32
    assert lib.moe_mx_quantize(-1, 64, p, q, r, None) == -1
    assert lib.moe_mx_quantize(4, 64, odd, q, r, None) == -2
    assert lib.moe_mx_quantize(4, 64, p, q, q, None) == -1                  # scales alias codes
    assert lib.moe_mx_quantize(0, 64, None, None, None, None) == 0          # empty
    mxf = lib.moe_expert_ffn_mxfp8
    s = moe.make_shape(16, 512, 8, 2, inter=512)
    b1, b2, b3, b4, b5 = (C.c_void_p(v) for v in (1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 22))
    assert mxf(C.byref(s), p, q, C.byref(lay), b1, b2, b3, b4, b5, p, 0, None) == -3       # no workspace
    assert mxf(C.byref(s), p, q, C.byref(lay), b1, b2, b3, None, b5, p, 1 << 30, None) == -1
    assert mxf(C.byref(s), p, C.c_void_p(12289), C.byref(lay), b1, b2, b3, b4, b5, p, 1 << 30, None) == -2
    assert mxf(C.byref(s), p, q, C.byref(lay), b1, b2, b3, b4, b1, p, 1 << 30, None) == -1  # y aliases a weight
    s_bad = moe.make_shape(16, 448, 8, 2, inter=512)                                      # H % 512
    assert mxf(C.byref(s_bad), p, q, C.byref(lay), b1, b2, b3, b4, b5, p, 1 << 30, None) == -4
    s_bad = moe.make_shape(16, 512, 8, 2, inter=1536 - 64)                                # I % 512
    assert mxf(C.byref(s_bad), p, q, C.byref(lay), b1, b2, b3, b4, b5, p, 1 << 30, None) == -4
    s = moe.make_shape(16, 64, 8, 2, inter=64, act_dtype=moe.MOE_DT_F32)
    assert lib.moe_expert_ffn(C.byref(s), p, C.byref(lay), p, p, p, None, p, 1 << 30, None) == -4  # fp32 FFN
    s = moe.make_shape(16, 64, 8, 2, inter=96)
    assert lib.moe_expert_ffn(C.byref(s), p, C.byref(lay), p, p, p, None, p, 1 << 30, None) == -4  # I % 64
    s = moe.make_shape(16, 64, 8, 2, inter=64)
    assert lib.moe_expert_ffn(C.byref(s), p, C.byref(lay), p, p, p, None, p, 16, None) == -3
    assert lib.moe_expert_ffn(C.byref(s), p, C.byref(lay), p, p, C.c_void_p(8192), odd, p, 1 << 30,
                              None) == -2                                 # misaligned gate_up
    assert lib.moe_expert_ffn(C.byref(s), p, C.byref(lay), p, p, C.c_void_p(8192), C.c_void_p(8192), p,
                              1 << 30, None) == -1                        # gate_up aliases y
    q, r = C.c_void_p(8192), C.c_void_p(12288)
    bwd = lib.moe_expert_ffn_bwd
    assert bwd(C.byref(s), p, p, None, C.byref(lay), p, p, q, r, C.c_void_p(16384), p, 16, None) == -3  # small ws
    assert bwd(C.byref(s), p, p, None, C.byref(lay), p, p, p, q, r, p, 1 << 30, None) == -1  # grad_x_perm aliases x_perm
    assert bwd(C.byref(s), p, p, None, C.byref(lay), p, p, q, r, r, p, 1 << 30, None) == -1  # the weight grads alias
    assert bwd(C.byref(s), p, p, None, C.byref(lay), p, p, q, odd, r, p, 1 << 30, None) == -2
    assert bwd(C.byref(s), p, p, None, None, p, p, q, r, C.c_void_p(16384), p, 1 << 30, None) == -1
    assert bwd(C.byref(s), p, p, None, C.byref(lay), p, p, q, None, r, p, 1 << 30, None) == -1  # null grad_w_gate_up
    assert bwd(C.byref(s), p, p, q, C.byref(lay), p, p, q, r, C.c_void_p(16384), p, 1 << 30, None) == -1  # gate_up
    s32 = moe.make_shape(16, 64, 8, 2, inter=64, act_dtype=moe.MOE_DT_F32)
    assert bwd(C.byref(s32), p, p, None, C.byref(lay), p, p, q, r, C.c_void_p(16384), p, 1 << 30, None) == -4
    assert lib.moe_combine(C.byref(s), p, p, C.byref(lay), p, None) == -1     # out aliases y
    assert lib.moe_combine(C.byref(s), odd, p, C.byref(lay), p, None) == -2
    assert lib.moe_dispatch_bwd(C.byref(s), p, C.byref(lay), p, None) == -1         # grad_x aliases grad_x_perm
    assert lib.moe_dispatch_bwd(C.byref(s), odd, C.byref(lay), p, None) == -2
    assert lib.moe_dispatch_bwd(C.byref(s), p, None, C.c_void_p(8192), None) == -1   # no layout
    assert lib.moe_combine_bwd(C.byref(s), p, p, p, C.byref(lay), p, p, None) == -1  # grad_y aliases


C_PROGRAM = r"""
#include "moe.h"
#include <stdio.h>
int main(void) {
  moe_shape s = {4096, 7168, 256, 8, 0, 0, 0, MOE_DT_BF16, 0, MOE_DROP_POSITION, 0};
  size_t b = 0;
  moe_status st = moe_workspace_size(MOE_OP_DISPATCH, &s, &b);
  s.capacity = 160;
  printf("%s %s %lld %lld %d\n", moe_version(), moe_status_string(st), (long long)moe_layout_rows(&s),
         (long long)(b > 0), (int)moe_dispatch(&s, 0, 0, 0, 0, 0, 0, 0, 0, 0));
  return st == MOE_OK ? 0 : 1;
}
"""


def test_header_is_plain_c_and_links(tmp_path, moe):
    """include/moe.h compiles as pedantic C99 with warnings as errors, and a C
    program links against the library and calls its host-side functions."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "t.c"
    src.write_text(C_PROGRAM)
    libdir = str(Path(moe.library_path).parent)
    exe = tmp_path / "t"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", str(ROOT / "include"),
                        str(src), "-L", libdir, "-lmoe_mi355x", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    version, status, rows, has_ws, null_layout = out.stdout.split()
    assert version == moe.lib.moe_version().decode() and status == "ok"
    assert int(rows) == 256 * 160 and has_ws == "1" and int(null_layout) == -1   # null layout: invalid argument
