"""Tensors past 2^32 elements: the per-token path (quantize, dequantize, STE
backward, dequantize backward) and the FP8 1 x 128 quantize / dequantize on
bf16 [1048640, 4096] (4,295,229,440 elements), where every element index
needs 64 bits and the FP8 block index leaves its 32-bit multiply-high form.
The input comes from torch's seeded device generator (N(0, 1)); rows on both
sides of element 2^32 and a random sample are checked against the oracle."""
import numpy as np
import pytest
import torch

from gpu_util import assert_same, from_dev, note

pytestmark = pytest.mark.gpu

ROWS, COLS = 1048640, 4096          # ROWS * COLS > 2^32; row 1048576 starts at element 2^32


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


@pytest.fixture(scope="module")
def big():
    if torch.cuda.get_device_properties(0).total_memory < 128 * 2**30:
        pytest.skip("needs a device with at least 128 GiB")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randn((ROWS, COLS), generator=g, dtype=torch.bfloat16, device="cuda")
    dy = torch.randn((ROWS, COLS), generator=g, dtype=torch.bfloat16, device="cuda")
    yield x, dy
    del x, dy
    torch.cuda.empty_cache()


def _rows():
    rng = np.random.default_rng(17)
    edge = [0, 1048575, 1048576, 1048577, ROWS - 1]
    return np.unique(np.concatenate([edge, rng.choice(ROWS, 24, replace=False)]))


def test_per_token_past_2_32(tq, orc, big):
    x, dy = big
    note("large per-token", tuple(x.shape))
    q, s, _ = tq.tq_quant_per_token(x, code="s8")
    y = tq.tq_dequant_per_token(q, x.shape, s, None, code="s8", out_dtype=torch.bfloat16)
    dx = tq.tq_quant_per_token_backward(x, dy, s, None, code="s8")
    dq = tq.tq_dequant_per_token_backward(dy, s)
    torch.cuda.synchronize()
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    xs, dys = from_dev(x[ri]), from_dev(dy[ri])
    oq, os_, _ = orc.quant_int(xs, "bf16", "token", code="s8")
    assert_same(from_dev(q[ri]), oq, "q")
    assert_same(from_dev(s[ri]), os_, "scale")
    assert_same(from_dev(y[ri]), orc.dequant_int(oq, "s8", xs.shape, "token", scale=os_, yt="bf16"), "dequant")
    assert_same(from_dev(dx[ri]), orc.quant_int_backward(xs, "bf16", "token", code="s8", scale=os_, dy=dys), "ste")
    assert_same(from_dev(dq[ri]), orc.dequant_int_backward(dys, "bf16", "token", scale=os_), "dq")
    del q, s, y, dx, dq


def test_fp8_1x128_past_2_32(tq, orc, big):
    x, _ = big
    note("large fp8 1x128", tuple(x.shape))
    q, s = tq.tq_quant_fp8_block(x, 1, 128)
    y = tq.tq_dequant_fp8_block(q, s, 1, 128, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _rows()
    ri = torch.from_numpy(rows).cuda()
    xs = from_dev(x[ri])
    oq, os_ = orc.quant_fp8_block(xs, "bf16", 1, 128)
    assert_same(from_dev(q[ri]), oq, "q")
    assert_same(from_dev(s[ri]), os_, "scale")
    assert_same(from_dev(y[ri]), orc.dequant_fp8_block(oq, 1, 128, os_, "bf16"), "dequant")
    del q, s, y
