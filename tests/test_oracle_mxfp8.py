"""Pins of the oracle's MXFP8 (E4M3 elements, one E8M0 scale per 32
elements along K; smile.llm.quant MxFp8, OCP MX v1.0 shared-scale rule).

The shared exponent is checked in closed form (floor(log2 amax) - 8, from
the binary32 exponent field, independent of the oracle's frexp), the
elements by brute-force nearest E4M3 search of x / X (exact: X is a power of
two), the STE mask and both backward products in numpy float32."""
import numpy as np
import pytest

import bruteforce as bf
import workloads


def _x_of(b):
    return np.ldexp(np.float64(1), b.astype(np.int64) - 127)


def test_e8m0_mx8_closed_form(orc):
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(5000).astype(np.float32)) * np.float32(2.0) ** rng.integers(-100, 100, 5000)
    amax = amax.astype(np.float32)
    b = orc.enc_e8m0_mx8(amax)
    e = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127      # floor(log2) of a normal value
    assert (b.astype(np.int64) == np.clip(e - 8 + 127, 0, 254)).all()
    r = amax.astype(np.float64) / _x_of(b)                                  # amax / X in [256, 512)
    assert ((r >= 256) & (r < 512)).all()
    assert orc.enc_e8m0_mx8(np.array([0.0], np.float32))[0] == 127
    assert orc.enc_e8m0_mx8(np.array([1.0], np.float32))[0] == 119
    assert orc.enc_e8m0_mx8(np.array([448.0], np.float32))[0] == 127
    assert orc.enc_e8m0_mx8(np.array([1e-40], np.float32))[0] == 0          # below 2^-119: clamped


@pytest.mark.parametrize("xt,sigma", [("f32", 1.0), ("bf16", 0.02), ("f16", 3.0), ("f32", 1e-37)])
def test_mxfp8_bruteforce(orc, xt, sigma):
    x = workloads.normal((6, 96), sigma, 11, xt)
    x[0, :32] = workloads.to_storage(np.zeros(32, np.float32), xt)              # all-zero block
    q, s = orc.quant_mxfp8(x, xt)
    xv = orc.widen(x, xt).astype(np.float32)
    blocks = xv.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    e = ((amax.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127
    want_s = np.where(amax == 0, 127, np.clip(e - 8 + 127, 0, 254)).astype(np.uint8)
    assert (s.ravel() == want_s).all()
    X = _x_of(want_s)[:, None]
    t = (blocks.astype(np.float64) / X).astype(np.float32)                     # exact: X is a power of two
    mags = bf.e4m3_magnitudes()
    want_q = bf.nearest_code(t, mags, 0x80).reshape(q.shape)
    assert (q == want_q).all()
    # the block max lands in the top binades of E4M3 ([256, 448], saturating)
    top = np.abs(t).max(axis=1)
    assert (top[(amax > 0) & (want_s > 0)] >= 256).all()          # unless the byte clamped at 0
    # dequant: val(q) * X in binary32, rounded once to the output type
    dec = np.zeros(256, np.float64)
    dec[:127], dec[128:255] = mags, -mags
    y = orc.dequant_mxfp8(q, s, "f32")
    yref = (dec[q].reshape(-1, 32) * X).astype(np.float32).reshape(q.shape)
    assert (y.view(np.uint32) == yref.view(np.uint32)).all()
    # STE and dequant backward
    dy = workloads.normal(x.shape, 1.0, 12, xt)
    dyv = orc.widen(dy, xt).astype(np.float32).reshape(-1, 32)
    mask = (np.abs(dec[q]) < 448).astype(np.float32).reshape(-1, 32)
    with np.errstate(over="ignore"):                                        # dy / 2^-127 may overflow to inf
        g = bf.mul32((dyv.astype(np.float64) / X).astype(np.float32), mask)
    dx = orc.quant_mxfp8_backward(x, xt, s, dy)
    assert (dx == workloads.to_storage(g.reshape(x.shape), xt)).all()
    dq = orc.dequant_mxfp8_backward(dy, xt, s)
    assert (dq == workloads.to_storage((dyv.astype(np.float64) * X).astype(np.float32).reshape(x.shape), xt)).all()


def test_mxfp8_rejects_ragged_k(orc):
    with pytest.raises(ValueError):
        orc.quant_mxfp8(np.zeros((2, 48), np.float32), "f32")
