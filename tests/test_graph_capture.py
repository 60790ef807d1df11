"""The library's calls inside a captured HIP graph (torch.cuda.graph): no call
allocates, synchronizes or records a memset node, so a captured sequence
replays the same kernels.  Each of several replays, separated by eager calls
on other data and by synchronizations, must reproduce the eager results bit
for bit; the captured outputs are overwritten between replays so that a
replay that did not run cannot pass."""
import pytest
import torch

import workloads
from gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def _bytes(t):
    return t.detach().contiguous().view(torch.uint8)


def _pipeline(tq, x, dy, xg, xt, w):
    """The per-token step, the dynamic per-tensor quantize (chunk partials,
    finalize and encode through a workspace), per-group u4, FP8 1x128, NVFP4
    with a dynamic global scale (amax pass, publish, encode) and its GEMM-layout
    transposes."""
    q, s, _ = tq.tq_quant_per_token(x, "s8")
    y = tq.tq_dequant_per_token(q, x.shape, s, code="s8", out_dtype=torch.bfloat16)
    dx = tq.tq_quant_per_token_backward(x, dy, s, code="s8")
    dq = tq.tq_dequant_per_token_backward(dy, s)
    qt, st, _ = tq.tq_quant_per_tensor(xt, "s8")
    qg, sg, zg = tq.tq_quant_per_group(xg, axis=-1, group_size=128, code="u4", symmetric=False)
    q8, s8 = tq.tq_quant_fp8_block(x, 1, 128)
    p, b, g = tq.tq_quant_fp4_block(w, "nvfp4")
    pt, bt = tq.tq_fp4_transpose_for_gemm(p, b, w.shape[0], w.shape[1], 16)
    return [q, s, y, dx, dq, qt, st, qg, sg, zg, q8, s8, p, b, g, pt, bt]


def test_graph_replays_match_eager(tq):
    note("graph capture: per-token step, per-tensor, per-group, FP8, NVFP4 + transposes")
    x = to_dev(workloads.normal((256, 4096), 1.0, 11, "bf16"), "bf16")
    dy = to_dev(workloads.normal((256, 4096), 1.0, 12, "bf16"), "bf16")
    xg = to_dev(workloads.normal((128, 4096), 0.02, 13, "f16"), "f16")
    xt = to_dev(workloads.normal((64, 256), 1.0, 14, "f32"))
    w = to_dev(workloads.normal((512, 1024), 0.02, 15, "bf16"), "bf16")
    other = [to_dev(workloads.normal(t.shape, 3.0, 20 + i, ft), ft)
             for i, (t, ft) in enumerate(((x, "bf16"), (dy, "bf16"), (xg, "f16"), (xt, "f32"), (w, "bf16")))]

    want = [_bytes(t).clone() for t in _pipeline(tq, x, dy, xg, xt, w)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _pipeline(tq, x, dy, xg, xt, w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _pipeline(tq, x, dy, xg, xt, w)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in outs:
            _bytes(t).fill_(0xA5)
        eager_other = _pipeline(tq, *other)        # eager work on other inputs between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, ref) in enumerate(zip(outs, want)):
            assert torch.equal(_bytes(t), ref), "replay %d, output %d differs from the eager result" % (rep, i)
        del eager_other
