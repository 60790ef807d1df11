"""GPU parity of the integer-code family (per-tensor / channel / token /
group; quantize, dequantize, STE backward, dequantize backward) against the
oracle, bit for bit.  Shapes cover every kernel path: team kernels
(L = 16..4096), the long-group kernel, column groups, the generic index path,
ragged tails, empty inputs and degenerate values.  The full-size workloads
are in test_parity_full.py."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH, assert_same, from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def nasty(shape, ft, seed):
    """Mixture of normal values, exact zeros (both signs), ties, tiny,
    subnormal (f32) and large magnitudes."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape).astype(np.float32)
    pick = rng.integers(0, 12, shape)
    v = np.where(pick == 0, np.float32(0.0), v)
    v = np.where(pick == 1, np.float32(-0.0), v)
    v = np.where(pick == 2, (rng.integers(-20, 20, shape) + 0.5).astype(np.float32), v)
    v = np.where(pick == 3, v * np.float32(2.0 ** -70), v)
    if ft == "f32":
        v = np.where(pick == 4, v * np.float32(1e-39), v)
    v = np.where(pick == 5, v * np.float32(1e4 if ft == "f16" else 1e20), v)
    return workloads.to_storage(v, ft)


def run_int_case(tq, orc, x, xt, gran, axis, g, code, sym, dy=None, rows_slice=None):
    """Quantize x on the GPU with granularity `gran`; compare q / scale / zp,
    dequant (to xt and f32), STE backward and dequant backward with the
    oracle."""
    shape = x.shape
    xd = to_dev(x, xt)
    note("case", gran, shape, xt, code, "sym" if sym else "asym", "axis", axis, "g", g)
    if gran == "token":
        q, s, z = tq.tq_quant_per_token(xd, code=code, symmetric=sym)
    elif gran == "channel":
        q, s, z = tq.tq_quant_per_channel(xd, axis=axis, code=code, symmetric=sym)
    elif gran == "group":
        q, s, z = tq.tq_quant_per_group(xd, axis=axis, group_size=g, code=code, symmetric=sym)
    else:
        q, s, z = tq.tq_quant_per_tensor(xd, code=code, symmetric=sym)
    oq, os_, oz = orc.quant_int(x, xt, gran, axis=axis, group_size=g, code=code, symmetric=sym)
    assert_same(from_dev(q), oq, "q")
    assert_same(from_dev(s).reshape(os_.shape), os_, "scale")
    if not sym:
        assert_same(from_dev(z).reshape(oz.shape), oz.view(np.uint8), "zero_point")
    # dequant
    for yt in {xt, "f32"}:
        if gran == "token":
            y = tq.tq_dequant_per_token(q, shape, s, z, code=code, out_dtype=TORCH[yt])
        elif gran == "channel":
            y = tq.tq_dequant_per_channel(q, shape, s, z, axis=axis, code=code, out_dtype=TORCH[yt])
        elif gran == "group":
            y = tq.tq_dequant_per_group(q, shape, s, z, axis=axis, group_size=g, code=code, out_dtype=TORCH[yt])
        else:
            y = tq.tq_dequant_per_tensor(q, shape, s, z, code=code, out_dtype=TORCH[yt])
        oy = orc.dequant_int(oq, code, shape, gran, axis, g, os_, oz, yt)
        assert_same(from_dev(y), oy, "dequant->" + yt)
    # STE backward and dequant backward
    if dy is None:
        dy = workloads.normal(shape, 1.0, 777, xt)
    dyd = to_dev(dy, xt)
    if gran == "token":
        dx = tq.tq_quant_per_token_backward(xd, dyd, s, z, code=code)
        dq = tq.tq_dequant_per_token_backward(dyd, s)
    elif gran == "channel":
        dx = tq.tq_quant_per_channel_backward(xd, dyd, s, z, axis=axis, code=code)
        dq = tq.tq_dequant_per_channel_backward(dyd, s, axis=axis)
    elif gran == "group":
        dx = tq.tq_quant_per_group_backward(xd, dyd, s, z, axis=axis, group_size=g, code=code)
        dq = tq.tq_dequant_per_group_backward(dyd, s, axis=axis, group_size=g)
    else:
        dx = tq.tq_quant_per_tensor_backward(xd, dyd, s, z, code=code)
        dq = tq.tq_dequant_per_tensor_backward(dyd, s)
    odx = orc.quant_int_backward(x, xt, gran, axis, g, code=code, symmetric=sym, scale=os_, zp=oz, dy=dy)
    assert_same(from_dev(dx), odx, "ste dx")
    odq = orc.dequant_int_backward(dy, xt, gran, axis, g, os_)
    assert_same(from_dev(dq), odq, "dequant backward dq")
    torch.cuda.synchronize()


TOKEN_CASES = [
    # rows, cols, xt, code, sym   (cols picks the kernel: team T = cols/8 or whole-wave W, long, generic)
    (37, 16, "bf16", "s8", True),
    (50, 32, "f16", "u8", False),
    (64, 64, "f32", "s8", True),
    (33, 128, "bf16", "u4", False),
    (20, 256, "f16", "s4", True),
    (9, 512, "bf16", "s8", True),
    (7, 1024, "f32", "u8", False),
    (5, 2048, "bf16", "s4", True),
    (65, 4096, "bf16", "s8", True),      # row-group kernel: 4 waves per 4096-element row
    (12, 4096, "f16", "u8", False),
    (10, 4096, "f32", "u4", False),
    (3, 4096, "bf16", "s4", True),
    (6, 7168, "bf16", "s8", True),
    (3, 4104, "f16", "u4", False),
    (11, 100, "f32", "s8", True),
    (4, 24, "bf16", "u8", False),
]


@pytest.mark.parametrize("rows,cols,xt,code,sym", TOKEN_CASES)
def test_per_token(tq, orc, rows, cols, xt, code, sym):
    x = workloads.normal((rows, cols), 1.5, rows * 1000 + cols, xt)
    run_int_case(tq, orc, x, xt, "token", 0, 0, code, sym)


@pytest.mark.parametrize("xt", ["bf16", "f32", "f16"])
def test_per_token_degenerate_values(tq, orc, xt):
    x = nasty((24, 512), xt, 5)
    x[3] = 0                                  # an all-zero row
    run_int_case(tq, orc, x, xt, "token", 0, 0, "s8", True, dy=nasty((24, 512), xt, 6))
    run_int_case(tq, orc, x, xt, "token", 0, 0, "u8", False, dy=nasty((24, 512), xt, 7))


GROUP_CASES = [
    # shape, xt, axis, g, code, sym
    ((40, 4096), "f16", 1, 128, "u4", False),
    ((17, 1024), "bf16", 1, 32, "s4", True),
    ((12, 512), "f32", 1, 64, "u8", False),
    ((8, 3, 256), "bf16", 2, 16, "s8", True),
    ((256, 96), "f16", 0, 64, "u4", False),       # column groups
    ((4, 64, 40), "bf16", 1, 16, "s8", True),     # column groups, 3-D
    ((6, 10, 6), "f32", 1, 5, "u4", False),        # generic (C % 8 != 0)
    ((3, 36), "f16", 1, 12, "u8", False),          # generic (L % 8 != 0)
    ((33,), "f32", 0, 1, "s8", True),              # group size 1
    # 4-bit dequantize variants: group map by division, with and without a
    # zero point, column groups without one, and a ragged last step
    ((9, 96), "f16", 1, 24, "u4", False),          # L = 24: not a power of two
    ((37, 480), "bf16", 1, 96, "s4", True),        # L = 96, symmetric
    ((130, 40), "f32", 0, 10, "s4", True),         # column groups, symmetric 4-bit
    ((35, 1024), "f16", 1, 128, "u4", False),      # g = 128 with a partial last step
]


@pytest.mark.parametrize("shape,xt,axis,g,code,sym", GROUP_CASES)
def test_per_group(tq, orc, shape, xt, axis, g, code, sym):
    x = workloads.normal(shape, 0.02, sum(shape) * 7 + g, xt)
    run_int_case(tq, orc, x, xt, "group", axis, g, code, sym)


CHANNEL_CASES = [
    ((64, 512), "bf16", 0, "s8", True),            # rows: team kernel
    ((300, 256), "f16", 1, "u8", False),           # columns
    ((5, 6, 40), "f32", 1, "s4", True),            # generic
    ((129,), "bf16", 0, "s8", True),               # 1-D: groups of one element
    ((16, 24), "f32", 1, "u4", False),             # columns, 4-bit
]


@pytest.mark.parametrize("shape,xt,axis,code,sym", CHANNEL_CASES)
def test_per_channel(tq, orc, shape, xt, axis, code, sym):
    x = workloads.normal(shape, 1.0, sum(shape) * 3 + axis, xt)
    run_int_case(tq, orc, x, xt, "channel", axis, 0, code, sym)


@pytest.mark.parametrize("numel,xt,code,sym", [(64 * 256, "f32", "s8", True), (2048, "f16", "u8", False),
                                               (32768, "bf16", "s4", True), (32776, "f32", "u4", False),
                                               (1 << 20, "bf16", "s8", True),
                                               (300_000, "f16", "u8", False), (1001, "f32", "s8", True),
                                               (1002, "bf16", "u4", False), (5 * (1 << 18), "f32", "s4", True)])
def test_per_tensor(tq, orc, numel, xt, code, sym):
    x = workloads.normal((numel,), 1.0, numel, xt)
    run_int_case(tq, orc, x, xt, "tensor", 0, 0, code, sym)


def test_per_tensor_workload_and_static_scale(tq, orc):
    x = workloads.make_input("c1_per_tensor_s8")
    dy = workloads.make_dy("c1_per_tensor_s8")
    run_int_case(tq, orc, x, "f32", "tensor", 0, 0, "s8", True, dy=dy)
    # static (caller-provided) scale and zero-point
    xd = to_dev(x.reshape(-1), "f32")
    s = torch.tensor([0.0123], dtype=torch.float32, device="cuda")
    q, _, _ = tq.tq_quant_per_tensor(xd, code="s8", scale=s)
    oq, _, _ = orc.quant_int(x.reshape(-1), "f32", "tensor", code="s8", scale=np.array([0.0123], np.float32))
    assert_same(from_dev(q), oq, "static q")
    z = torch.tensor([3], dtype=torch.uint8, device="cuda")
    q, _, _ = tq.tq_quant_per_tensor(xd, code="u8", symmetric=False, scale=s, zero_point=z)
    oq, _, _ = orc.quant_int(x.reshape(-1), "f32", "tensor", code="u8", symmetric=False,
                             scale=np.array([0.0123], np.float32), zp=np.array([3], np.uint8))
    assert_same(from_dev(q), oq, "static asym q")


def test_empty_inputs(tq):
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    q, s, z = tq.tq_quant_per_token(x)
    assert q.numel() == 0 and s.numel() == 0
    q, s, z = tq.tq_quant_per_group(x, axis=1, group_size=128, code="u4")
    assert q.shape == (0, 64)
