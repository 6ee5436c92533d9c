"""Pins for the oracle's MXFP8 quantisation and MXFP8 dispatch.  CPU only.

The format is MXFP8 as the OCP "Microscaling (MX) Formats Specification" v1.0
defines it (the reading of the MORI pull request's FP8 dispatch with per-token
scales and of the ROCm Megatron MXFP8 recipe): 32-element blocks, one E8M0
scale 2^s per block with s = floor(log2(amax)) - 8 clipped to [-127, 127],
elements FP8 E4M3 (bias 7, no infinities, largest finite 448) rounded to
nearest with ties to even and clamped to +-448.

Pins: closed-form code values, a round trip over every code, midpoints between
neighbouring codes, torch's own float8_e4m3fn conversion (a library routine) on
every finite bf16 value in range, and a pure-Python quantiser that derives each
code from floor(log2) and Python's half-to-even round() -- a different
algorithm from the oracle's search over the code table.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from parity_util import every_value_at_every_scale

RNG = np.random.default_rng(2024)


# --------------------------------------------------------- pure-Python reference

def py_e4m3(v: float) -> int:
    """E4M3 code of v from the grid spacing: magnitudes in [2^e, 2^(e+1)) (e >= -6)
    sit on multiples of 2^(e-3), smaller ones on multiples of 2^-9."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = min(abs(v), 448.0)
    if a == 0.0:
        return sign
    e = max(math.frexp(a)[1] - 1, -6)
    step = 2.0 ** (e - 3)
    val = round(a / step) * step          # Python round(): halves to the even integer
    if val < 2.0 ** -6:
        return sign | int(val / 2.0 ** -9)
    e2 = math.frexp(val)[1] - 1
    return sign | ((e2 + 7) << 3) | (int(val / 2.0 ** (e2 - 3)) - 8)


def py_mx_block(vals):
    """(scale code, element codes) of one 32-element block of Python floats."""
    amax = max(abs(v) for v in vals)
    s = -127 if amax == 0.0 else min(max(math.frexp(amax)[1] - 1 - 8, -127), 127)
    return s + 127, [py_e4m3(v / 2.0 ** s) for v in vals]


def all_finite_bf16() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]


def bf16_f64(b: np.ndarray) -> np.ndarray:
    return mi.bf16_bits_to_f32(b).astype(np.float64)


# ------------------------------------------------------------------ E4M3 codes

def test_e4m3_decode_closed_forms():
    codes = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x77, 0x7E, 0x80, 0xB8, 0xFE], np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.875, 240.0, 448.0, -0.0, -1.0, -448.0]
    got = oracle.e4m3_decode(codes)
    assert got.tolist() == want
    assert np.signbit(got[9])
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_values_ascend_and_round_trip():
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert (np.diff(vals) > 0).all()
    assert (oracle.e4m3_encode(vals) == codes).all()
    assert (oracle.e4m3_encode(-vals[1:]) == codes[1:] | 0x80).all()
    assert oracle.e4m3_encode(np.array([-0.0]))[0] == 0x80


def test_e4m3_midpoints_go_to_even_code():
    codes = np.arange(0x7E, dtype=np.int64)
    lo, hi = oracle.e4m3_decode(codes.astype(np.uint8)), oracle.e4m3_decode((codes + 1).astype(np.uint8))
    mid = (lo + hi) / 2
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert (oracle.e4m3_encode(mid) == even).all()
    assert (oracle.e4m3_encode(np.nextafter(mid, np.inf)) == codes + 1).all()
    assert (oracle.e4m3_encode(np.nextafter(mid, -np.inf)) == codes).all()


def test_e4m3_clamps_to_largest_finite():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 511.0, 1e30, -1e30])
    assert oracle.e4m3_encode(v).tolist() == [0x7E] * 7 + [0xFE]


def test_e4m3_matches_torch_float8_on_every_bf16():
    """torch's float8_e4m3fn conversion rounds to nearest-even and gives NaN from
    464 up; below that it must agree with the oracle on every finite bf16."""
    b = all_finite_bf16()
    v = bf16_f64(b)
    v = v[np.abs(v) < 464.0]
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (oracle.e4m3_encode(v) == want).all()


def test_e4m3_matches_python_grid_rounding():
    b = all_finite_bf16()
    v = bf16_f64(b)[::7]
    v = np.concatenate([v, RNG.uniform(-500, 500, 2000), RNG.standard_normal(2000) * 2.0 ** -7])
    want = np.array([py_e4m3(float(t)) for t in v], np.uint8)
    assert (oracle.e4m3_encode(v) == want).all()


# -------------------------------------------------------------------- MX scale

def test_mx_scale_closed_form():
    """A block whose largest magnitude lies in [2^p, 2^(p+1)) has scale code
    clip(p - 8, -127, 127) + 127; an all-zero block has code 0."""
    ps = list(range(-133, 128))
    x = np.zeros((len(ps) + 1, 32), np.float32)
    for i, p in enumerate(ps):
        top = np.float32(2.0 ** p * (1.0 + RNG.uniform(0, 0.99)))
        x[i, :] = top * RNG.uniform(-1, 1, 32).astype(np.float32)
        x[i, RNG.integers(32)] = -top if i % 2 else top
    xb = mi.f32_to_bf16_bits(x)
    amax = np.abs(bf16_f64(xb)).max(axis=1)
    q, sc = oracle.mx_quantize(xb)
    want = [int(np.clip(math.frexp(a)[1] - 1 - 8, -127, 127)) + 127 if a > 0 else 0 for a in amax]
    assert sc[:, 0].tolist() == want
    assert sc[-1, 0] == 0 and (q[-1] == 0).all()


def test_mx_block_property_largest_element():
    """With an unclipped scale the largest element lands in [256, 512) before
    rounding, so its code decodes to a value in [256, 448]."""
    x = mi.f32_to_bf16_bits((RNG.standard_normal((64, 256)) * np.exp(RNG.uniform(-20, 20, (64, 1)))).astype(np.float32))
    q, sc = oracle.mx_quantize(x)
    dq = np.abs(oracle.e4m3_decode(q)).reshape(64, 8, 32).max(axis=2)
    assert ((dq >= 256) & (dq <= 448)).all()
    assert (sc > 0).all()


def test_mx_quantize_matches_python_blocks():
    rows, h = 6, 128
    x = (RNG.standard_normal((rows, h)) * np.exp(RNG.uniform(-8, 8, (rows, h // 32)).repeat(32, axis=1))).astype(np.float32)
    x[0, :32] = 0.0                                    # zero block
    x[1, 32:64] = 2.0 ** -130 * RNG.integers(-3, 4, 32)  # bf16 subnormals: clipped scale
    x[2, 64:96] = 3.0e38 * RNG.uniform(-1, 1, 32)      # near the bf16 maximum
    x[3, :] = -0.0
    xb = mi.f32_to_bf16_bits(x)
    q, sc = oracle.mx_quantize(xb)
    v = bf16_f64(xb)
    for r in range(rows):
        for blk in range(h // 32):
            code, els = py_mx_block([float(t) for t in v[r, 32 * blk:32 * blk + 32]])
            assert sc[r, blk] == code, (r, blk)
            assert q[r, 32 * blk:32 * blk + 32].tolist() == els, (r, blk)


def test_mx_dequantize_error_bound():
    """Each element of an unclipped block is within half a grid step of its value:
    2^(s + e - 4) for magnitudes in [2^(s+e), 2^(s+e+1)), e >= -6, unless clamped
    to 448 * 2^s."""
    x = mi.f32_to_bf16_bits((RNG.standard_normal((32, 512)) * 3).astype(np.float32))
    q, sc = oracle.mx_quantize(x)
    v = bf16_f64(x)
    dq = oracle.mx_dequantize(q, sc)
    s = np.repeat(sc.astype(np.int64) - 127, 32, axis=1)
    a = np.abs(v) / 2.0 ** s
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    bound = np.where(a > 448.0, np.abs(v) - 448.0 * 2.0 ** s, 2.0 ** (s + e - 4))
    assert (np.abs(dq - v) <= bound).all()


# ---------------------------------------------------------------- MXFP8 dispatch

@pytest.mark.parametrize("capacity,row_align", [(0, 0), (3, 0), (0, 4)])
def test_dispatch_mxfp8_rows_are_quantised_token_rows(capacity, row_align):
    n, h, e, k = 13, 96, 5, 2
    x = mi.f32_to_bf16_bits(RNG.standard_normal((n, h)).astype(np.float32))
    idx = np.stack([RNG.choice(e, k, replace=False) for _ in range(n)]).astype(np.int32)
    idx[4, 1] = -1
    w = RNG.uniform(0, 1, (n, k)).astype(np.float32)
    lay = oracle.layout(idx, e, capacity=capacity, row_align=row_align)
    pq, ps, wp = oracle.dispatch_mxfp8(x, k, lay, w)
    v = bf16_f64(x)
    for a in range(n * k):
        r = lay["assign_row"][a]
        if r < 0:
            continue
        code_els = [py_mx_block([float(t) for t in v[a // k, 32 * b:32 * b + 32]]) for b in range(h // 32)]
        assert ps[r].tolist() == [c for c, _ in code_els]
        assert pq[r].tolist() == [c for _, els in code_els for c in els]
        assert wp[r] == w.flat[a]
    end = int(lay["expert_offsets"][-1])
    for r in range(lay["rows"]):
        if lay["row_src"][r] < 0 and r < end:
            assert not pq[r].any() and not ps[r].any() and wp[r] == 0


# ------------------------------------------------------------ MXFP8 expert FFN

def _mx(shape, scale_sigma, rng):
    x = mi.f32_to_bf16_bits((rng.standard_normal(shape) * scale_sigma).astype(np.float32))
    q, s = oracle.mx_quantize(x.reshape(-1, shape[-1]))
    return q.reshape(shape), s.reshape(shape[:-1] + (shape[-1] // 32,))


def test_expert_ffn_mxfp8_matches_composed_pinned_steps():
    """The MXFP8 FFN oracle equals its definition composed from independently
    pinned pieces: MX dequantisation, numpy fp64 matmuls, the bf16 rounding, the
    MX quantisation of the intermediate."""
    rng = np.random.default_rng(77)
    e, h, inter, rows = 3, 64, 64, 20
    xq, xs = _mx((rows, h), 1.0, rng)
    gq, gs = _mx((e, 2 * inter, h), 0.1, rng)
    dq, ds = _mx((e, h, inter), 0.1, rng)
    lay = {"expert_offsets": np.array([0, 6, 6, 17], np.int32), "tokens_per_expert": np.array([6, 0, 11], np.int32)}
    got, ex = oracle.expert_ffn_mxfp8_rows(np.arange(rows), xq, xs, lay, gq, gs, dq, ds)
    x = oracle.mx_dequantize(xq, xs)
    wgu = oracle.mx_dequantize(gq.reshape(-1, h), gs.reshape(-1, h // 32)).reshape(e, 2 * inter, h)
    wd = oracle.mx_dequantize(dq.reshape(-1, inter), ds.reshape(-1, inter // 32)).reshape(e, h, inter)
    for r in range(rows):
        x_e = {0: 0, 1: 0, 2: 0, 3: 0, 4: 0, 5: 0}.get(r, 2 if 6 <= r < 17 else -1)
        assert ex[r] == x_e
        if x_e < 0:
            assert not got[r].any()
            continue
        gu = wgu[x_e] @ x[r]
        g, u = gu[:inter], gu[inter:]
        a = oracle.bf16_round_array(g / (1 + np.exp(-g)) * u)
        aq, as_ = oracle.mx_quantize(a[None, :])
        y = wd[x_e] @ oracle.mx_dequantize(aq, as_)[0]
        np.testing.assert_array_equal(got[r], oracle.bf16_round_array(y))


def test_expert_ffn_mxfp8_zero_gate():
    """Zero gate weights give exactly zero rows (silu(0) = 0)."""
    rng = np.random.default_rng(5)
    e, h, inter, rows = 2, 64, 32, 8
    xq, xs = _mx((rows, h), 1.0, rng)
    gq, gs = _mx((e, 2 * inter, h), 0.1, rng)
    dq, ds = _mx((e, h, inter), 0.1, rng)
    gq[:, :inter] = 0
    lay = {"expert_offsets": np.array([0, 4, 8], np.int32), "tokens_per_expert": np.array([4, 4], np.int32)}
    got, _ = oracle.expert_ffn_mxfp8_rows(np.arange(rows), xq, xs, lay, gq, gs, dq, ds)
    assert not got.any()


def test_every_value_at_every_scale_covers_the_codes():
    x = every_value_at_every_scale()
    _, sc = oracle.mx_quantize(x)
    assert set(np.unique(sc).tolist()) == set(range(247))           # scale codes 0 .. 246
    mag = x & 0x7FFF
    assert ((mag >> 7) != 0xFF).all()                                # finite only
