"""GPU parity of per-tensor fake quantization (round trip and its
straight-through backward) and of dynamic-range quantization against the
oracle, bit for bit.  Fake quantization is covered on every per-tensor path:
the one-launch small kernel (dynamic, numel % 8 == 0, up to 32768 elements),
the single-workgroup encode (up to 65536), the two-pass reduce + encode
(larger), the scalar path (numel % 8 != 0) and static scales."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same, from_dev, note, to_dev
from test_parity_int import nasty

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def run_fake(tq, orc, x, xt, code, sym, scale=None, zp=None, dy=None):
    note("fake case", x.shape, xt, code, "sym" if sym else "asym", "static" if scale is not None else "dynamic")
    xd = to_dev(x, xt)
    sd = None if scale is None else torch.tensor(np.atleast_1d(scale).astype(np.float32), device="cuda")
    zd = None if zp is None else torch.from_numpy(np.atleast_1d(zp).copy()).cuda()
    y, s, z = tq.tq_fake_quant_per_tensor(xd, code=code, symmetric=sym, scale=sd, zero_point=zd)
    oy, os_, oz = orc.fake_quant_per_tensor(x, xt, code, symmetric=sym, scale=scale, zp=zp)
    assert_same(from_dev(s), os_, "scale")
    if not sym:
        assert_same(from_dev(z), oz.view(np.uint8), "zero_point")
    assert_same(from_dev(y), oy, "round trip")
    if dy is None:
        dy = workloads.normal(x.shape, 1.0, 77, xt)
    dx = tq.tq_fake_quant_per_tensor_backward(xd, to_dev(dy, xt), s, z, code=code)
    assert_same(from_dev(dx), orc.fake_quant_per_tensor_backward(x, xt, dy, os_, oz, code=code, symmetric=sym),
                "backward")


@pytest.mark.parametrize("shape,xt,code,sym", [
    ((64, 256), "f32", "s8", True),          # small one-launch kernel
    ((16, 2048), "bf16", "u8", False),       # single-workgroup encode
    ((4096, 4096), "bf16", "s8", True),      # two-pass reduce + encode
    ((513, 1031), "f16", "s8", False),       # scalar path (numel % 8 != 0)
    ((3, 5), "f32", "s4", True),
    ((40, 64), "f16", "u4", False),
])
def test_fake_quant(tq, orc, shape, xt, code, sym):
    x = workloads.normal(shape, 1.0, shape[0] * 31 + shape[1], xt)
    run_fake(tq, orc, x, xt, code, sym)


@pytest.mark.parametrize("xt", ["f32", "bf16", "f16"])
def test_fake_quant_degenerate_values(tq, orc, xt):
    x = nasty((96, 333), xt, 5)
    run_fake(tq, orc, x, xt, "s8", True, dy=nasty((96, 333), xt, 6))
    run_fake(tq, orc, x, xt, "u8", False, dy=nasty((96, 333), xt, 7))
    run_fake(tq, orc, np.zeros((8, 8), workloads.to_storage(np.zeros(1, np.float32), xt).dtype), xt, "s8", True)


def test_fake_quant_static_scales(tq, orc):
    x = workloads.normal((256, 1024), 1.0, 9, "bf16")
    run_fake(tq, orc, x, "bf16", "s8", True, scale=np.float32(0.0125))                      # many clamped codes
    run_fake(tq, orc, x, "bf16", "u8", False, scale=np.float32(0.01), zp=np.array([120], np.uint8))
    run_fake(tq, orc, x, "bf16", "s8", False, scale=np.float32(3e-39), zp=np.array([-5], np.int8))  # tiny scale
    run_fake(tq, orc, x[:255, :1001].copy(), "bf16", "s8", True, scale=np.float32(0.02))    # scalar path


def test_fake_quant_full_size(tq, orc):
    """bf16 [8192, 4096] activations (the per-token workload's input) through
    the per-tensor round trip, every element against the oracle."""
    x = workloads.make_input("c2_per_token_s8")
    run_fake(tq, orc, x, "bf16", "s8", True, dy=workloads.make_dy("c2_per_token_s8"))


def test_fake_quant_empty(tq):
    x = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    y, s, _ = tq.tq_fake_quant_per_tensor(x)
    assert y.numel() == 0


@pytest.mark.parametrize("shape,xt,mode,scope,axis,code", [
    ((6, 4096), "bf16", "symmetric", "token", 0, "s8"),
    ((2, 5, 256), "f32", "asymmetric", "token", 0, "u8"),
    ((64, 256), "f16", "symmetric", "tensor", 0, "s4"),
    ((70000,), "bf16", "asymmetric", "tensor", 0, "u8"),
    ((48, 96), "f32", "asymmetric", "channel", 1, "u4"),
    ((48, 96), "bf16", "symmetric", "channel", 0, "s8"),
])
def test_dynamic_range(tq, orc, shape, xt, mode, scope, axis, code):
    note("dynamic range", shape, xt, mode, scope, axis, code)
    x = workloads.normal(shape, 2.0, len(shape) * 1000 + shape[-1], xt)
    q, s, z = tq.tq_dynamic_range_quantize(to_dev(x, xt), mode, scope, code, axis)
    oq, os_, oz = orc.dynamic_range_quantize(x, xt, mode, scope, code, axis)
    assert_same(from_dev(q), oq, "q")
    assert_same(from_dev(s).reshape(os_.shape), os_, "scale")
    if mode == "asymmetric":
        assert_same(from_dev(z).reshape(oz.shape), oz.view(np.uint8), "zero_point")
    else:
        assert z is None


def test_dynamic_range_rejects_bad_mode(tq):
    x = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError):
        tq.tq_dynamic_range_quantize(x, "symmetric", "token", "u8")
