"""GPU parity of the binary64 family (f64 inputs computed in binary64):
quantize, dequantize, STE backward and dequantize backward at every
granularity against the oracle, bit for bit, including the per-tensor
two-pass reduction, ragged shapes, static scales and degenerate values."""
import numpy as np
import pytest
import torch

from gpu_util import assert_same, from_dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def run_f64(tq, orc, x, gran, axis, g, code, sym, dy=None, scale=None, zp=None):
    note("f64 case", x.shape, gran, axis, g, code, "sym" if sym else "asym", "static" if scale is not None else "")
    xd = torch.from_numpy(x).cuda()
    sd = None if scale is None else torch.from_numpy(np.asarray(scale, np.float64)).cuda()
    zd = None if zp is None else torch.from_numpy(np.asarray(zp)).cuda()
    q, s, z = tq.tq_quant_f64(xd, gran, axis, g, code=code, symmetric=sym, scale=sd, zero_point=zd)
    oq, os_, oz = orc.quant_f64(x, gran, axis, g, code=code, symmetric=sym, scale=scale, zp=zp)
    assert_same(from_dev(s).reshape(os_.shape).view(np.uint64), os_.view(np.uint64), "scale")
    if not sym:
        assert_same(from_dev(z).reshape(oz.shape), oz.view(np.uint8), "zero_point")
    assert_same(from_dev(q), oq, "codes")
    y = tq.tq_dequant_f64(q, x.shape, s, z, gran, axis, g, code=code)
    assert_same(from_dev(y).view(np.uint64), orc.dequant_f64(oq, code, x.shape, gran, axis, g, os_, oz).view(np.uint64),
                "dequant")
    if dy is None:
        dy = np.random.default_rng(5).standard_normal(x.shape)
    dyd = torch.from_numpy(dy).cuda()
    dx = tq.tq_quant_f64_backward(xd, dyd, s, z, gran, axis, g, code=code)
    want = orc.quant_f64_backward(x, gran, axis, g, code=code, symmetric=sym, scale=os_, zp=oz, dy=dy)
    assert_same(from_dev(dx).view(np.uint64), want.view(np.uint64), "ste")
    dq = tq.tq_dequant_f64_backward(dyd, s, gran, axis, g)
    assert_same(from_dev(dq).view(np.uint64), orc.dequant_f64_backward(dy, gran, axis, g, os_).view(np.uint64), "dq")


@pytest.mark.parametrize("shape,gran,axis,g,code,sym", [
    ((64, 4096), "token", 0, 0, "s8", True),
    ((33, 100), "token", 0, 0, "u8", False),
    ((2, 3, 40), "token", 0, 0, "s4", True),
    ((48, 256), "group", 1, 128, "u4", False),
    ((64, 24), "group", 0, 16, "s8", False),
    ((12, 34), "channel", 0, 0, "s8", True),
    ((12, 34), "channel", 1, 0, "u8", False),
    ((1000,), "tensor", 0, 0, "s8", True),
    ((2048, 4096), "tensor", 0, 0, "u8", False),    # two-pass reduction (chunk partials + finalize)
    ((16, 12), "token", 0, 0, "s8", False),         # 8-element vectors that straddle rows
    ((8, 60), "group", 1, 12, "s4", True),          # ... and groups along the last axis
    ((30, 400), "token", 0, 0, "u8", False),        # one-pass rows at 64, 128, 256, 512 and 1024
    ((40, 1000), "token", 0, 0, "u8", False),       # threads, rows not a multiple of the
    ((6, 4096), "group", 1, 2048, "u4", False),     # workgroup's reach
    ((20, 2050), "token", 0, 0, "s4", True),
    ((4, 6000), "token", 0, 0, "u8", False),
])
def test_f64(tq, orc, shape, gran, axis, g, code, sym):
    x = np.random.default_rng(len(shape) * 100 + shape[-1]).standard_normal(shape) * 2.5
    run_f64(tq, orc, x, gran, axis, g, code, sym)


def test_f64_degenerate_and_static(tq, orc):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, 64))
    x[0] = 0.0
    x[1, :] = -0.0
    x[2, :] = np.arange(64) * 0.5 - 16.0            # exact ties k + 1/2 for scale 1 rows
    x[3, :] = 1e-310                                # binary64 subnormals
    x[4, :8] = 1e300
    run_f64(tq, orc, x, "token", 0, 0, "s8", True)
    run_f64(tq, orc, x, "token", 0, 0, "u8", False)
    run_f64(tq, orc, x, "token", 0, 0, "s8", True, scale=np.full(16, 0.0125))        # many clamped codes
    run_f64(tq, orc, x, "token", 0, 0, "u8", False, scale=np.full(16, 0.01), zp=np.full(16, 120, np.uint8))


def test_f64_empty(tq):
    x = torch.empty((0, 8), dtype=torch.float64, device="cuda")
    q, s, _ = tq.tq_quant_f64(x, "token")
    assert q.numel() == 0


def _near_ties(rng, s, n):
    """n elements next to (k + 1/2) * s, |k| <= 126: the tie itself and up to
    two binary64 steps either side."""
    x = (rng.integers(-126, 126, size=n).astype(np.float64) + 0.5) * s
    for _ in range(2):
        step = rng.integers(-1, 2, size=n)
        x = np.where(step > 0, np.nextafter(x, np.inf), np.where(step < 0, np.nextafter(x, -np.inf), x))
    return x


def test_f64_quotient_edges(tq, orc):
    """The quantize kernels divide by two FMA corrections of x * RN(1/s) when
    2^-400 <= |s| <= 2^400 (and, for static scales, |x| <= 2^600), otherwise
    by IEEE division: quotients at and next to the ties k + 1/2, scales on
    both sides of the guard, huge, infinite and subnormal elements."""
    rng = np.random.default_rng(21)
    # dynamic per-token (one pass): amax fixes s = amax / 127, the rest sit at ties of s
    amax = rng.uniform(1.0, 2.0, size=6) * 2.0 ** np.array([-40, -3, 0, 5, 300, -398])
    x = np.stack([_near_ties(rng, a / 127.0, 1024) for a in amax])
    x[:, 7] = amax
    run_f64(tq, orc, x, "token", 0, 0, "s8", True)
    # static per-tensor scales: fast (2^-300, exactly 2^-400, 1.5) and slow (2^-401, 2^401)
    for s, sub in ((2.0 ** -300, False), (2.0 ** -400, True), (1.5, True), (2.0 ** -401, True), (2.0 ** 401, False)):
        x = _near_ties(rng, s, 8 * 1024).reshape(8, 1024)
        if sub:
            x[0, :4] = [5e-324, -5e-324, 1e-310, -2.0 ** -1000]
        x[1, :6] = [np.inf, -np.inf, 2.0 ** 601, -2.0 ** 600, 1e308, -1e308]
        run_f64(tq, orc, x, "tensor", 0, 0, "s8", True, scale=np.array([s]))
        run_f64(tq, orc, x, "tensor", 0, 0, "u8", False, scale=np.array([s]), zp=np.array([128], np.uint8))
