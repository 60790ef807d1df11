"""GPU parity at the full workload sizes, on every output element.

Each workload is run through the same calls, at the same shapes, that the
benchmark times -- quantize, dequantize, STE backward and dequantize
backward (and the GEMM-layout transposes of the FP4 weight) -- and the whole
of every output is compared with the oracle bit for bit.  The oracle calls
of one workload run in parallel host threads (each is a ctypes call that
releases the interpreter lock); their arithmetic is unchanged.

Workloads (seeded, see workloads/__init__.py):
  per-token s8      bf16 [8192, 4096] N(0,1), 41 outlier columns x20
  per-group u4 g128 f16 [11008, 4096] N(0, 0.02), asymmetric
  FP8 1x128         bf16 [4096, 7168] N(0,1)
  FP8 128x128       bf16 [7168, 7168] N(0, 0.02)
  NVFP4 / MXFP4     bf16 [14336, 4096] N(0, 0.02)
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same, from_dev, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def _parallel(*calls):
    with ThreadPoolExecutor(max_workers=len(calls)) as ex:
        futs = [ex.submit(fn, *args) for fn, *args in calls]
        return [f.result() for f in futs]


def test_full_per_token_s8(tq, orc):
    note("full per-token s8 bf16 [8192, 4096]")
    x = workloads.make_input("c2_per_token_s8")
    dy = workloads.make_dy("c2_per_token_s8")
    xd, dyd = to_dev(x, "bf16"), to_dev(dy, "bf16")
    q, s, _ = tq.tq_quant_per_token(xd, code="s8")
    y = tq.tq_dequant_per_token(q, x.shape, s, None, code="s8", out_dtype=torch.bfloat16)
    dx = tq.tq_quant_per_token_backward(xd, dyd, s, None, code="s8")
    dq = tq.tq_dequant_per_token_backward(dyd, s)
    q, s, y, dx, dq = map(from_dev, (q, s, y, dx, dq))
    oq, os_, _ = orc.quant_int(x, "bf16", "token", code="s8")
    assert_same(q, oq, "q")
    assert_same(s, os_, "scale")
    oy, odx, odq = _parallel(
        (orc.dequant_int, oq, "s8", x.shape, "token", 0, 0, os_, None, "bf16"),
        (lambda: orc.quant_int_backward(x, "bf16", "token", code="s8", scale=os_, dy=dy),),
        (orc.dequant_int_backward, dy, "bf16", "token", 0, 0, os_))
    assert_same(y, oy, "dequant")
    assert_same(dx, odx, "ste")
    assert_same(dq, odq, "dq")


def test_full_per_group_u4_g128(tq, orc):
    note("full per-group u4 g128 f16 [11008, 4096]")
    w = workloads.make_input("c3_per_group_u4_g128")
    dy = workloads.normal(w.shape, 1.0, 302, "f16")
    wd, dyd = to_dev(w, "f16"), to_dev(dy, "f16")
    q, s, z = tq.tq_quant_per_group(wd, axis=1, group_size=128, code="u4", symmetric=False)
    y = tq.tq_dequant_per_group(q, w.shape, s, z, axis=1, group_size=128, code="u4", out_dtype=torch.float16)
    dx = tq.tq_quant_per_group_backward(wd, dyd, s, z, axis=1, group_size=128, code="u4")
    dq = tq.tq_dequant_per_group_backward(dyd, s, axis=1, group_size=128)
    q, s, z, y, dx, dq = map(from_dev, (q, s, z, y, dx, dq))
    oq, os_, oz = orc.quant_int(w, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    assert_same(q, oq, "q")
    assert_same(s, os_, "scale")
    assert_same(z, oz, "zp")
    oy, odx, odq = _parallel(
        (orc.dequant_int, oq, "u4", w.shape, "group", 1, 128, os_, oz, "f16"),
        (lambda: orc.quant_int_backward(w, "f16", "group", 1, 128, code="u4", symmetric=False, scale=os_,
                                        zp=oz, dy=dy),),
        (orc.dequant_int_backward, dy, "f16", "group", 1, 128, os_))
    assert_same(y, oy, "dequant")
    assert_same(dx, odx, "ste")
    assert_same(dq, odq, "dq")


@pytest.mark.parametrize("name,block", [("c4_fp8_act_1x128", (1, 128)), ("c4_fp8_weight_128x128", (128, 128))])
def test_full_fp8_block(tq, orc, name, block):
    br, bc = block
    x = workloads.make_input(name)
    note("full FP8", name, x.shape)
    dy = workloads.make_dy(name)
    xd, dyd = to_dev(x, "bf16"), to_dev(dy, "bf16")
    q, s = tq.tq_quant_fp8_block(xd, br, bc)
    y = tq.tq_dequant_fp8_block(q, s, br, bc, out_dtype=torch.bfloat16)
    dx = tq.tq_quant_fp8_block_backward(xd, dyd, s, br, bc)
    dq = tq.tq_dequant_fp8_block_backward(dyd, s, br, bc)
    q, s, y, dx, dq = map(from_dev, (q, s, y, dx, dq))
    oq, os_ = orc.quant_fp8_block(x, "bf16", br, bc)
    assert_same(q, oq, "q")
    assert_same(s, os_, "scale")
    oy, odx, odq = _parallel(
        (orc.dequant_fp8_block, oq, br, bc, os_, "bf16"),
        (orc.quant_fp8_block_backward, x, "bf16", br, bc, os_, dy),
        (orc.dequant_fp8_block_backward, dy, "bf16", br, bc, os_))
    assert_same(y, oy, "dequant")
    assert_same(dx, odx, "ste")
    assert_same(dq, odq, "dq")


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_full_fp4(tq, orc, kind):
    """Dynamic per-tensor scale for NVFP4 (two passes), then every output
    and the GEMM-layout transposes of codes and block scales."""
    gs = 16 if kind == "nvfp4" else 32
    w = workloads.make_input("c5_fp4_weight")
    note("full", kind, w.shape)
    dy = workloads.make_dy("c5_fp4_weight")
    wd, dyd = to_dev(w, "bf16"), to_dev(dy, "bf16")
    p, b, g = tq.tq_quant_fp4_block(wd, kind)
    y = tq.tq_dequant_fp4_block(p, b, g, kind, out_dtype=torch.bfloat16)
    dx = tq.tq_quant_fp4_block_backward(wd, dyd, b, g, kind)
    dq = tq.tq_dequant_fp4_block_backward(dyd, b, g, kind)
    pt, bt = tq.tq_fp4_transpose_for_gemm(p, b, w.shape[0], w.shape[1], gs)
    P, B, y, dx, dq, PT, BT = map(from_dev, (p, b, y, dx, dq, pt, bt))
    op, ob, og = orc.quant_fp4_block(w, "bf16", kind)
    assert_same(P, op, "packed")
    assert_same(B, ob, "block scales")
    sg = og[0] if kind == "nvfp4" else np.float32(1.0)
    if kind == "nvfp4":
        assert_same(from_dev(g), og, "global scale")
    oy, odx, odq, (opt, obt) = _parallel(
        (orc.dequant_fp4_block, op, ob, sg, kind, "bf16"),
        (orc.quant_fp4_block_backward, w, "bf16", ob, sg, kind, dy),
        (orc.dequant_fp4_block_backward, dy, "bf16", ob, sg, kind),
        (orc.fp4_transpose_for_gemm, op, ob, w.shape[0], w.shape[1], gs))
    assert_same(y, oy, "dequant")
    assert_same(dx, odx, "ste")
    assert_same(dq, odq, "dq")
    assert_same(PT, opt, "packed^T")
    assert_same(BT, obt, "scales^T")
