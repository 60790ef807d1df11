"""The library holds no state between calls: two host threads, each on its
own HIP stream, call the quantize path concurrently (ctypes releases the
interpreter lock during each call, so the calls really overlap on the host
and their kernels on the device) and every result equals the serial one."""
import threading

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


def _work(tq, x, dy, w):
    q, s, _ = tq.tq_quant_per_token(x, "s8")
    y = tq.tq_dequant_per_token(q, x.shape, s, code="s8", out_dtype=torch.bfloat16)
    dx = tq.tq_quant_per_token_backward(x, dy, s, code="s8")
    qt, st, _ = tq.tq_quant_per_tensor(x, "s8")
    p, b, g = tq.tq_quant_fp4_block(w, "nvfp4")
    return [t.contiguous().view(torch.uint8) for t in (q, s, y, dx, qt, st, p, b, g)]


def test_two_threads_two_streams(tq):
    note("concurrency: two host threads, two streams")
    inputs = []
    for i in range(2):
        x = to_dev(workloads.normal((512, 4096), 1.0, 31 + i, "bf16"), "bf16")
        dy = to_dev(workloads.normal((512, 4096), 1.0, 41 + i, "bf16"), "bf16")
        w = to_dev(workloads.normal((1024, 2048), 0.02, 51 + i, "bf16"), "bf16")
        inputs.append((x, dy, w))
    want = [[t.clone() for t in _work(tq, *inp)] for inp in inputs]
    torch.cuda.synchronize()

    results = [[None] * 8 for _ in range(2)]
    errors = []

    def worker(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for it in range(8):
                    results[k][it] = _work(tq, *inputs[k])
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        for it in range(8):
            for i, (got, ref) in enumerate(zip(results[k][it], want[k])):
                assert torch.equal(got, ref), "thread %d, iteration %d, output %d" % (k, it, i)
