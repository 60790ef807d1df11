"""Pins of the oracle's fake quantization (per-tensor floating-point round
trip and its straight-through backward) and of dynamic-range quantization
(data-derived range at a chosen scope, then quantize).

Checked against: the hand-worked per-token example (one row, scale 1, so the
round trip returns the codes and the backward returns dy's masked values),
the brute-force re-derivation of per-tensor / per-token / per-channel
quantization (exhaustive nearest code, numpy float32 steps), and closed-form
properties (the round trip is within half a step of x, is idempotent under a
static scale, and lands on the grid (k - zp) * scale).
"""
import zlib

import numpy as np
import pytest

import bruteforce as bf
import workloads
from test_oracle_quant import _narrow, _read_worked, _unpack, _values, bf_nearest_int, bf_quant_int


def test_worked_example_round_trip(orc):
    x, s, q, dy, dx = _read_worked("per_token_s8_worked.txt")
    x = np.array([float(v) for v in x], np.float32)
    dy = np.array([float(v) for v in dy], np.float32)
    y, so, _ = orc.fake_quant_per_tensor(x, "f32", "s8")
    assert so[0] == float(s[0]) == 1.0
    want = np.array([float(v) for v in q], np.float32)          # (q - 0) * 1
    assert (y.view(np.uint32) == want.view(np.uint32)).all()
    g = orc.fake_quant_per_tensor_backward(x, "f32", dy, so)
    wdx = np.array([float(v) for v in dx], np.float32)            # dy / 1 masked
    assert (g.view(np.uint32) == wdx.view(np.uint32)).all()


CASES = [((4, 6), "f32", "s8", True), ((3, 40), "bf16", "s8", True), ((2, 24), "f16", "u8", False),
         ((5, 8), "bf16", "u4", False), ((7,), "f32", "s4", True), ((3, 11), "f16", "s8", False)]


@pytest.mark.parametrize("shape,xt,code,sym", CASES)
def test_fake_quant_bruteforce(orc, shape, xt, code, sym):
    seed = zlib.crc32(repr((shape, xt, code, sym)).encode())
    x = workloads.normal(shape, 1.0, seed, xt)
    qmin, qmax = orc.default_q_range(code, sym)
    y, s, z = orc.fake_quant_per_tensor(x, xt, code, symmetric=sym)
    xv = _values(x, xt)
    codes, bs, bz = bf_quant_int(xv, shape, "tensor", 0, 0, qmin, qmax, sym)
    assert s[0].view(np.uint32) == bs[0].view(np.uint32)
    if not sym:
        assert int(z[0]) == int(bz[0])
    want = _narrow(bf.mul32(np.float32(codes - bz[0]), bs[0]), xt)
    assert (y == want).all()
    # backward: dy where qmin < q < qmax, else a zero with dy's sign
    dy = workloads.normal(shape, 1.0, seed + 1, xt)
    dx = orc.fake_quant_per_tensor_backward(x, xt, dy, s, z, code=code, symmetric=sym)
    dyv = _values(dy, xt)
    dref = bf.mul32(dyv, ((codes > qmin) & (codes < qmax)).astype(np.float32))
    assert (dx == _narrow(dref, xt)).all()


def test_fake_quant_static_scale_clamps_and_is_idempotent(orc):
    x = workloads.normal((8, 64), 1.0, 5, "f32")
    s = np.float32(0.0125)                 # |x| / s reaches far beyond 127: many clamped codes
    y, _, _ = orc.fake_quant_per_tensor(x, "f32", "s8", scale=s)
    assert np.abs(y).max() == np.float32(127 * s)
    inside = np.abs(x) < np.float32(126.5) * s
    assert inside.sum() > 100 and (~inside).sum() > 20
    assert (np.abs(y[inside] - x[inside]) <= s / 2 * (1 + 2 ** -20)).all()
    # on the grid k * s, and a second round trip changes nothing
    k = np.rint(y / s)
    assert (bf.mul32(np.float32(k), s) == y).all()
    y2, _, _ = orc.fake_quant_per_tensor(y, "f32", "s8", scale=s)
    assert (y2.view(np.uint32) == y.view(np.uint32)).all()
    # backward mask: zero exactly where the code was clamped or hit +-127
    dy = np.ones_like(x)
    dx = orc.fake_quant_per_tensor_backward(x, "f32", dy, np.array([s], np.float32))
    assert ((dx == 1.0) == (np.abs(k) < 127)).all()


def test_fake_quant_asymmetric_static_zero_point(orc):
    x = workloads.normal((4, 32), 1.5, 6, "bf16")
    s, zp = np.float32(0.01), 120
    y, _, _ = orc.fake_quant_per_tensor(x, "bf16", "u8", symmetric=False, scale=s, zp=np.array([zp], np.uint8))
    c = bf_nearest_int(bf.div32(_values(x, "bf16").ravel(), s), 0, 255, zp)
    assert (c == 0).any() and (c == 255).any()                 # both clamp bounds are reached
    want = _narrow(bf.mul32(np.float32(c - zp), s), "bf16").reshape(x.shape)
    assert (y == want).all()


@pytest.mark.parametrize("shape,xt,mode,scope,axis,code", [
    ((6, 32), "bf16", "symmetric", "token", 0, "s8"),
    ((6, 32), "f32", "asymmetric", "token", 0, "u8"),
    ((2, 3, 16), "f16", "symmetric", "tensor", 0, "s4"),
    ((5, 12), "f32", "asymmetric", "channel", 1, "u4"),
    ((5, 12), "bf16", "symmetric", "channel", 0, "s8"),
])
def test_dynamic_range_bruteforce(orc, shape, xt, mode, scope, axis, code):
    seed = zlib.crc32(repr((shape, xt, mode, scope, axis, code)).encode())
    x = workloads.normal(shape, 2.0, seed, xt)
    sym = mode == "symmetric"
    q, s, z = orc.dynamic_range_quantize(x, xt, mode, scope, code, axis)
    # the code's default range for the mode: s8 -> [-127, 127] / [-128, 127], u8 -> [0, 255] ...
    qmin, qmax = {("s8", True): (-127, 127), ("s8", False): (-128, 127), ("u8", False): (0, 255),
                  ("s4", True): (-7, 7), ("s4", False): (-8, 7), ("u4", False): (0, 15)}[(code, sym)]
    codes, bs, bz = bf_quant_int(_values(x, xt), shape, scope, axis, 0, qmin, qmax, sym)
    assert (_unpack(q, code, shape) == codes).all()
    assert (s.ravel().view(np.uint32) == bs.view(np.uint32)).all()
    if not sym:
        assert (z.ravel().astype(np.int32) == bz).all()
    else:
        assert z is None


def test_dynamic_range_rejects_unsigned_symmetric(orc):
    with pytest.raises(ValueError):
        orc.dynamic_range_quantize(np.zeros((2, 8), np.float32), "f32", "symmetric", "token", "u8")
