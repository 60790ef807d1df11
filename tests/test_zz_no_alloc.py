"""The allocation-free FP4 block quantize (tq_quant_fp4_block_noalloc, for
callers that cannot allocate: graph capture, serving loops) against the
workspace version tq_quant_fp4_block, bit for bit, through the C ABI: two
calls in a row on one device, the second on a smaller tensor, so the second
reads only what it wrote into the library's scratch array."""
import ctypes

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


def _noalloc(tq, x, kind, global_scale=None):
    rows, k = x.shape
    gs = 16 if kind == "nvfp4" else 32
    packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    bs = torch.empty((rows, k // gs), dtype=torch.uint8, device=x.device)
    static = global_scale is not None
    sg = None
    if kind == "nvfp4":
        sg = global_scale.clone() if static else torch.full((1,), -1.0, dtype=torch.float32, device=x.device)
    rc = tq._lib.tq_quant_fp4_block_noalloc(
        ctypes.c_void_p(x.data_ptr()), tq.FTYPE[x.dtype], rows, k, tq.FP4_KIND[kind],
        ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(bs.data_ptr()),
        None if sg is None else ctypes.c_void_p(sg.data_ptr()), int(static),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, tq._lib.tq_status_str(rc)
    return packed, bs, sg


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_noalloc_matches_workspace_version(tq, orc, kind):
    big = workloads.make_input("c5_fp4_weight")                       # [14336, 4096]: 1024 partials
    small = workloads.normal((300, 4096), 0.02, 77, "bf16")           # 152 partials
    for name, x in (("c5 [14336,4096]", big), ("[300,4096]", small)):
        note("noalloc", kind, name)
        xd = to_dev(x, "bf16")
        p1, b1, g1 = tq.tq_quant_fp4_block(xd, kind)
        p2, b2, g2 = _noalloc(tq, xd, kind)
        torch.cuda.synchronize()
        assert_same(from_dev(p2), from_dev(p1), "packed " + name)
        assert_same(from_dev(b2), from_dev(b1), "block scales " + name)
        if kind == "nvfp4":
            assert_same(from_dev(g2), from_dev(g1), "global scale " + name)
    op, ob, og = orc.quant_fp4_block(small, "bf16", kind)
    assert_same(from_dev(p2), op, "packed vs oracle")
    assert_same(from_dev(b2), ob, "block scales vs oracle")
    if kind == "nvfp4":
        assert_same(from_dev(g2), og, "global scale vs oracle")


def test_noalloc_static_global_and_errors(tq):
    x = to_dev(workloads.normal((64, 512), 0.02, 5, "bf16"), "bf16")
    sg = torch.tensor([3.1e-5], dtype=torch.float32, device="cuda")
    p1, b1, _ = tq.tq_quant_fp4_block(x, "nvfp4", global_scale=sg)
    p2, b2, g2 = _noalloc(tq, x, "nvfp4", global_scale=sg)
    torch.cuda.synchronize()
    assert_same(from_dev(p2), from_dev(p1), "packed static")
    assert_same(from_dev(b2), from_dev(b1), "block scales static")
    assert from_dev(g2)[0] == np.float32(3.1e-5)
    f = tq._lib.tq_quant_fp4_block_noalloc
    assert f(None, 2, 4, 32, 0, None, None, None, 0, None) == tq.TQ_ERR_INVALID       # null pointers
    assert f(ctypes.c_void_p(x.data_ptr()), 2, 4, 24, 0, ctypes.c_void_p(p1.data_ptr()),
             ctypes.c_void_p(b1.data_ptr()), ctypes.c_void_p(sg.data_ptr()), 0, None) == tq.TQ_ERR_INVALID  # k % 16
    assert f(None, 2, 0, 32, 0, None, None, None, 0, None) == 0                         # empty: nothing to do
