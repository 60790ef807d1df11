"""GPU parity of the row-strided quantizers (per-token integer codes and FP8
1 x bc blocks reading a column slice of a wider matrix in place) against the
oracle on the dense rows, bit for bit, and against the contiguous calls."""
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


def _slice(rows, ld, off, cols, xt, seed):
    full = workloads.normal((rows, ld), 1.0, seed, xt)
    dev = to_dev(full, xt)
    return dev[:, off:off + cols], np.ascontiguousarray(full[:, off:off + cols])


@pytest.mark.parametrize("rows,ld,off,cols,xt,code,sym", [
    (64, 7168, 1024, 4096, "bf16", "s8", True),     # 4-wave row kernel
    (40, 384, 128, 128, "f16", "u4", False),        # team kernel, 4-bit asymmetric
    (9, 1024, 16, 1000, "f32", "s8", True),         # long-row kernel (1000 columns)
    (17, 4096, 2048, 2048, "bf16", "s4", True),
    (5, 96, 8, 64, "f16", "u8", False),
])
def test_per_token_strided(tq, orc, rows, ld, off, cols, xt, code, sym):
    note("per-token strided", rows, ld, off, cols, xt, code, sym)
    view, dense = _slice(rows, ld, off, cols, xt, rows * 31 + cols)
    assert view.stride(0) == ld
    q, s, z = tq.tq_quant_per_token_strided(view, code=code, symmetric=sym)
    oq, os_, oz = orc.quant_int(dense, xt, "token", code=code, symmetric=sym)
    assert_same(from_dev(q), oq, "codes")
    assert_same(from_dev(s), os_, "scale")
    if not sym:
        assert_same(from_dev(z), oz.view(np.uint8), "zero_point")
    q2, s2, _ = tq.tq_quant_per_token(view.contiguous(), code=code, symmetric=sym)
    assert_same(from_dev(q), from_dev(q2), "strided == contiguous")


@pytest.mark.parametrize("rows,ld,off,cols,bc,xt", [
    (32, 7168, 3072, 4096, 128, "bf16"),
    (7, 512, 64, 256, 32, "f16"),
    (5, 2048, 512, 1024, 512, "f32"),
    (3, 160, 16, 64, 16, "bf16"),
])
def test_fp8_rows_strided(tq, orc, rows, ld, off, cols, bc, xt):
    note("fp8 strided", rows, ld, off, cols, bc, xt)
    view, dense = _slice(rows, ld, off, cols, xt, rows * 7 + cols)
    q, s = tq.tq_quant_fp8_rows_strided(view, bc)
    oq, os_ = orc.quant_fp8_block(dense, xt, 1, bc)
    assert_same(from_dev(q), oq, "codes")
    assert_same(from_dev(s), os_, "scales")


def test_strided_errors(tq):
    x = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tq.TQError):                        # 100 bf16 = 200-byte rows: not 16-byte aligned strides
        tq.tq_quant_per_token_strided(x[:, :96])
    with pytest.raises(tq.TQError):                        # 12 columns: not a multiple of 8
        tq.tq_quant_per_token_strided(torch.zeros((4, 64), dtype=torch.float32, device="cuda")[:, :12])
    with pytest.raises(tq.TQError):                        # block of 96 columns: no row kernel for it
        tq.tq_quant_fp8_rows_strided(torch.zeros((4, 384), dtype=torch.float32, device="cuda")[:, :192], 96)
