"""GPU parity of MXFP8 (E4M3 elements, E8M0 scale per 32 elements):
quantize, dequantize, STE backward and dequantize backward against the
oracle, bit for bit, on ragged wave tails, degenerate values (zeros, ties,
tiny blocks whose scale byte clamps at 0, saturation) and a full-size
[4096, 7168] bf16 activation."""
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


def run_mx8(tq, orc, x, xt, dy=None):
    note("mxfp8 case", x.shape, xt)
    xd = to_dev(x, xt)
    q, b = tq.tq_quant_mxfp8(xd)
    oq, ob = orc.quant_mxfp8(x, xt)
    assert_same(from_dev(b), ob, "scales")
    assert_same(from_dev(q), oq, "codes")
    for yt in {xt, "f32"}:
        y = tq.tq_dequant_mxfp8(q, b, out_dtype=TORCH[yt])
        assert_same(from_dev(y), orc.dequant_mxfp8(oq, ob, yt), "dequant->" + yt)
    if dy is None:
        dy = workloads.normal(x.shape, 1.0, 99, xt)
    dyd = to_dev(dy, xt)
    assert_same(from_dev(tq.tq_quant_mxfp8_backward(xd, dyd, b)), orc.quant_mxfp8_backward(x, xt, ob, dy), "ste")
    assert_same(from_dev(tq.tq_dequant_mxfp8_backward(dyd, b)), orc.dequant_mxfp8_backward(dy, xt, ob), "dq")


@pytest.mark.parametrize("shape,xt", [((64, 4096), "bf16"), ((37, 160), "f16"), ((3, 32), "f32"),
                                      ((129, 96), "bf16"), ((1, 2048 + 32), "f32")])
def test_mxfp8(tq, orc, shape, xt):
    run_mx8(tq, orc, workloads.normal(shape, 1.0, shape[0] * 13 + shape[1], xt), xt)


@pytest.mark.parametrize("xt", ["bf16", "f32", "f16"])
def test_mxfp8_degenerate_values(tq, orc, xt):
    x = nasty((32, 256), xt, 31)
    x[0, :64] = 0
    tiny = 1e-38 if xt != "f16" else 1e-7
    x[1, 32:64] = workloads.to_storage(np.full(32, tiny, np.float32), xt)
    x[2, :32] = workloads.to_storage(np.linspace(-448, 448, 32).astype(np.float32), xt)
    dy = nasty((32, 256), xt, 32)
    if xt == "f32":
        # keep dy / X finite where the mask is zero (inf * 0 would be a NaN)
        dy = np.where(np.abs(dy) > 1e20, np.float32(1.0), dy)
    run_mx8(tq, orc, x, xt, dy=dy)


def test_mxfp8_full_size_sampled(tq, orc):
    x = workloads.make_input("c4_fp8_act_1x128")
    q, b = tq.tq_quant_mxfp8(to_dev(x, "bf16"))
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(8).choice(4096, 40, replace=False)]))
    oq, ob = orc.quant_mxfp8(np.ascontiguousarray(x[rows]), "bf16")
    assert_same(from_dev(q)[rows], oq, "codes")
    assert_same(from_dev(b)[rows], ob, "scales")


def test_mxfp8_rejects_ragged_k(tq):
    with pytest.raises(tq.TQError):
        tq.tq_quant_mxfp8(torch.zeros((2, 48), dtype=torch.float32, device="cuda"))
