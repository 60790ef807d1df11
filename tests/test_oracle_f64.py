"""Pins of the oracle's binary64 family (f64 inputs computed in binary64).

Re-derived on tiny tensors with exact rationals: the quotient x / scale is
formed as an exact Fraction and rounded once to binary64 by Python's
correctly rounded float(Fraction); codes are then found by exhaustive
nearest-integer search (ties to even).  Closed forms: the element at amax
maps to +-qmax (symmetric), the round trip stays within half a step, and a
second quantization of the dequantized values with the same scale returns
the same codes."""
import zlib
from fractions import Fraction

import numpy as np
import pytest

from test_oracle_quant import _unpack, bf_groups, bf_nearest_int


def rn64(fr):
    return float(fr)            # correctly rounded Fraction -> binary64


def bf_quant_f64(x, shape, gran, axis, g, qmin, qmax, sym):
    groups = bf_groups(shape, gran, axis, g)
    flat = x.ravel()
    scale = np.zeros(len(groups))
    zp = np.zeros(len(groups), np.int64)
    codes = np.zeros(flat.size, np.int64)
    for gid, m in groups:
        v = flat[m]
        if sym:
            s = rn64(Fraction(float(np.abs(v).max())) / qmax)
            s = 1.0 if s == 0 else s
            z = 0
        else:
            mn, mx = min(float(v.min()), 0.0), max(float(v.max()), 0.0)
            s = rn64(Fraction(rn64(Fraction(mx) - Fraction(mn))) / (qmax - qmin))
            s = 1.0 if s == 0 else s
            t = rn64(Fraction(mn) / Fraction(s))
            z = int(np.clip(qmin - round(t), qmin, qmax))      # round(): ties to even on the binary64 value
        scale[gid], zp[gid] = s, z
        t = np.array([rn64(Fraction(float(a)) / Fraction(s)) for a in v])
        codes[m] = bf_nearest_int(t, qmin, qmax, z)
    return codes.reshape(shape), scale, zp


CASES = [((3, 16), "token", 0, 0, "s8", True), ((2, 24), "token", 0, 0, "u8", False),
         ((4, 6), "tensor", 0, 0, "s8", True), ((5, 8), "channel", 1, 0, "u4", False),
         ((4, 32), "group", 1, 8, "s4", True), ((6, 4), "group", 0, 3, "u8", False)]


@pytest.mark.parametrize("shape,gran,axis,g,code,sym", CASES)
def test_f64_bruteforce(orc, shape, gran, axis, g, code, sym):
    seed = zlib.crc32(repr((shape, gran, axis, g, code, sym)).encode())
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * 3.0
    qmin, qmax = orc.default_q_range(code, sym)
    q, s, z = orc.quant_f64(x, gran, axis, g, code=code, symmetric=sym)
    codes, bs, bz = bf_quant_f64(x, shape, gran, axis, g, qmin, qmax, sym)
    assert (s.ravel() == bs).all()
    if not sym:
        assert (z.ravel().astype(np.int64) == bz).all()
    assert (_unpack(q, code, shape) == codes).all()
    groups = bf_groups(shape, gran, axis, g)
    y = orc.dequant_f64(q, code, shape, gran, axis, g, s, z)
    yref = np.zeros(x.size)
    for gid, m in groups:
        yref[m] = [rn64(Fraction(int(c) - int(bz[gid])) * Fraction(bs[gid])) for c in codes.ravel()[m]]
    assert (y.ravel() == yref).all()
    dy = rng.standard_normal(shape)
    dx = orc.quant_f64_backward(x, gran, axis, g, code=code, qmin=qmin, qmax=qmax, symmetric=sym, scale=s, zp=z,
                                dy=dy)
    dref = np.zeros(x.size)
    for gid, m in groups:
        c = codes.ravel()[m]
        for e, cc in zip(m, c):
            qd = rn64(Fraction(float(dy.ravel()[e])) / Fraction(bs[gid]))
            dref[e] = qd * (1.0 if qmin < cc < qmax else 0.0)
    assert (dx.ravel().view(np.uint64) == dref.view(np.uint64)).all()
    dq = orc.dequant_f64_backward(dy, gran, axis, g, s)
    dqref = np.zeros(x.size)
    for gid, m in groups:
        dqref[m] = [rn64(Fraction(float(dy.ravel()[e])) * Fraction(bs[gid])) for e in m]
    assert (dq.ravel() == dqref).all()


def test_f64_closed_forms(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 64)) * 5
    q, s, _ = orc.quant_f64(x, "token", code="s8")
    c = _unpack(q, "s8", x.shape)
    am = np.abs(x).argmax(axis=1)
    assert (np.abs(c[np.arange(16), am]) == 127).all()
    y = orc.dequant_f64(q, "s8", x.shape, "token", scale=s)
    assert (np.abs(y - x) <= s[:, None] / 2 * (1 + 1e-12)).all()
    q2, _, _ = orc.quant_f64(y, "token", code="s8", scale=s)
    assert (q2 == q).all()
