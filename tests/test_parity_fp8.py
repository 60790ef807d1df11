"""GPU parity of the FP8 E4M3 block family (1x128 activation groups,
128x128 weight tiles and other block shapes; quantize, dequantize, STE,
dequantize backward) against the oracle, bit for bit, plus a dense check of
the E4M3 conversion itself."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import TORCH, assert_same, from_dev, note, to_dev
from test_parity_int import nasty

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def run_fp8(tq, orc, x, xt, br, bc, dy=None):
    rows, cols = x.shape
    note("fp8 case", x.shape, xt, (br, bc))
    xd = to_dev(x, xt)
    q, s = tq.tq_quant_fp8_block(xd, br, bc)
    oq, os_ = orc.quant_fp8_block(x, xt, br, bc)
    assert_same(from_dev(q), oq, "q")
    assert_same(from_dev(s), os_, "scale")
    for yt in {xt, "f32"}:
        y = tq.tq_dequant_fp8_block(q, s, br, bc, out_dtype=TORCH[yt])
        assert_same(from_dev(y), orc.dequant_fp8_block(oq, br, bc, os_, yt), "dequant->" + yt)
    if dy is None:
        dy = workloads.normal(x.shape, 1.0, 4242, xt)
    dyd = to_dev(dy, xt)
    dx = tq.tq_quant_fp8_block_backward(xd, dyd, s, br, bc)
    assert_same(from_dev(dx), orc.quant_fp8_block_backward(x, xt, br, bc, os_, dy), "ste")
    dq = tq.tq_dequant_fp8_block_backward(dyd, s, br, bc)
    assert_same(from_dev(dq), orc.dequant_fp8_block_backward(dy, xt, br, bc, os_), "dq")


@pytest.mark.parametrize("shape,xt,block", [
    ((96, 7168), "bf16", (1, 128)),
    ((33, 256), "f16", (1, 128)),
    ((16, 512), "f32", (1, 16)),
    ((8, 1024), "bf16", (1, 32)),
    ((4, 512), "bf16", (1, 64)),
    ((4, 1024), "bf16", (1, 256)),
    ((3, 1024), "f16", (1, 512)),
    ((384, 512), "bf16", (128, 128)),
    ((128, 384), "f32", (128, 128)),
    ((192, 256), "f16", (64, 128)),
    ((128, 192), "bf16", (64, 64)),
    ((6, 40), "bf16", (2, 8)),           # generic blocks
    ((6, 36), "f32", (3, 12)),           # cols % 8 != 0: generic elementwise
    ((2, 1024), "bf16", (1, 1024)),      # generic (block wider than 512)
])
def test_fp8_blocks(tq, orc, shape, xt, block):
    x = workloads.normal(shape, 2.0, shape[0] * 31 + block[1], xt)
    run_fp8(tq, orc, x, xt, *block)


@pytest.mark.parametrize("xt", ["bf16", "f32"])
def test_fp8_degenerate_values(tq, orc, xt):
    x = nasty((256, 256), xt, 11)
    x[:128, :128] = 0
    run_fp8(tq, orc, x, xt, 1, 128, dy=nasty((256, 256), xt, 12))
    run_fp8(tq, orc, x, xt, 128, 128, dy=nasty((256, 256), xt, 13))


def test_e4m3_conversion_dense(tq, orc):
    """Blocks whose max |x| is 448 have scale 1 exactly, so their codes are
    the E4M3 encodings of the inputs themselves: a dense sweep of binary32
    values in [2^-12, 448] (every 61st pattern, both signs) plus midpoints."""
    lo, hi = np.float32(2.0 ** -12).view(np.uint32), np.float32(448.0).view(np.uint32)
    v = np.arange(lo, hi + 1, 61, dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 1e-30, -1e-30], np.float32)])
    n = (v.size + 126) // 127 * 127
    v = np.concatenate([v, np.zeros(n - v.size, np.float32)]).reshape(-1, 127)
    x = np.concatenate([np.full((v.shape[0], 1), 448.0, np.float32), v], axis=1)
    q, s = tq.tq_quant_fp8_block(to_dev(x, "f32"), 1, 128)
    assert (from_dev(s) == 1.0).all()
    assert_same(from_dev(q), orc.enc_e4m3(x), "E4M3 codes")


@pytest.mark.parametrize("shape,xt,block", [
    ((5, 7000), "bf16", (1, 128)),        # ragged K: last 1x128 group has 88 elements
    ((200, 330), "f32", (128, 128)),      # partial tiles on both edges
    ((130, 256), "bf16", (128, 128)),     # one partial block row
    ((7, 9), "f16", (4, 4)),              # odd everything (scalar element path)
    ((3, 100), "bf16", (8, 64)),          # block taller than the tensor
])
def test_fp8_partial_tiles(tq, orc, shape, xt, block):
    run_fp8(tq, orc, workloads.normal(shape, 2.0, shape[0] * 7 + shape[1], xt), xt, *block)


@pytest.mark.parametrize("shape,xt,static", [
    ((64, 256), "bf16", None),             # one launch (<= 65536 elements)
    ((4096, 7168), "bf16", None),          # two passes (c4 activation size)
    ((333, 777), "f16", None),             # scalar path, two passes
    ((16, 1024), "f32", 0.004),            # static: many saturated codes
    ((5, 7), "bf16", 1e-3),                # static, scalar path
    ((300, 1000), "bf16", 0.02),           # static, vectors in a partial last step
    ((257, 1024), "f16", None),            # two passes, partial last step of the encode
])
def test_fp8_per_tensor(tq, orc, shape, xt, static):
    note("fp8 per tensor", shape, xt, static)
    x = workloads.normal(shape, 1.0, shape[0] + 3 * shape[1], xt)
    sd = None if static is None else torch.tensor([static], dtype=torch.float32, device="cuda")
    q, s = tq.tq_quant_fp8_per_tensor(to_dev(x, xt), sd)
    oq, os_ = orc.quant_fp8_per_tensor(x, xt, None if static is None else np.float32(static))
    assert_same(from_dev(s), os_, "scale")
    assert_same(from_dev(q), oq, "codes")
    for yt in {xt, "f32"}:
        y = tq.tq_dequant_fp8_per_tensor(q, s, out_dtype=TORCH[yt])
        want = orc.dequant_fp8_block(oq.reshape(1, -1), 1, oq.size, os_.reshape(1, 1), yt).reshape(shape)
        assert_same(from_dev(y), want, "load->" + yt)


def test_fp8_per_tensor_degenerate(tq, orc):
    x = nasty((40, 100), "f32", 44)
    for static in (None, np.float32(2.5e-3)):
        sd = None if static is None else torch.tensor([static], device="cuda")
        q, s = tq.tq_quant_fp8_per_tensor(to_dev(x, "f32"), sd)
        oq, os_ = orc.quant_fp8_per_tensor(x, "f32", static)
        assert_same(from_dev(q), oq, "codes")
        assert_same(from_dev(s), os_, "scale")
