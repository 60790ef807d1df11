"""Randomized GPU parity sweeps.  The integer-code family: 64 seeded cases
draw the granularity, the rank (1-3), the shape (ragged and odd sizes
included), the axis, the group size among the divisors of that axis, the
input type, the code, symmetric or zero-point, and plain or "nasty" values;
every output (codes, scales, zero-points, dequantize to two types, STE
backward, dequantize backward) must equal the oracle's bits.  The draws are
printed before each case, so a failure names its case."""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import note
from test_parity_int import nasty, run_int_case

pytestmark = pytest.mark.gpu

GRANS = ("token", "channel", "group", "tensor")
FTS = ("f32", "f16", "bf16")


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def _draw(rng):
    gran = GRANS[rng.integers(len(GRANS))]
    ndim = int(rng.integers(1, 4)) if gran != "token" else int(rng.integers(2, 4))
    dims = [int(rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 64, 96, 128, 200, 256, 384]))
            for _ in range(ndim)]
    while int(np.prod(dims)) > 65536:
        dims[int(rng.integers(ndim))] = max(1, dims[int(rng.integers(ndim))] // 4)
    sym = bool(rng.integers(2))
    code = str(rng.choice(["s8", "s4"] if sym else ["u8", "u4", "s8", "s4"]))
    if code in ("s4", "u4") and dims[-1] % 2:
        dims[-1] += 1                          # 4-bit codes pack pairs along the last axis
    axis, g = 0, 0
    if gran in ("channel", "group"):
        axis = int(rng.integers(ndim))
    if gran == "group":
        n = dims[axis]
        divs = [d for d in range(1, n + 1) if n % d == 0]
        g = int(rng.choice(divs))
    return gran, tuple(dims), axis, g, code, sym, FTS[rng.integers(len(FTS))], bool(rng.integers(2))


def test_random_integer_cases(tq, orc):
    rng = np.random.default_rng(20261203)
    for case in range(64):
        gran, shape, axis, g, code, sym, xt, bad = _draw(rng)
        note("random case", case)
        seed = 9000 + case
        x = nasty(shape, xt, seed) if bad else workloads.normal(shape, 1.5, seed, xt)
        if xt == "f16":                        # keep the large f16 draws finite (infinities are out of contract)
            h = x.view(np.float16)
            h[np.isinf(h)] = np.copysign(np.float16(60000.0), h[np.isinf(h)])
        dy = workloads.normal(shape, 1.0, seed + 1, xt)
        run_int_case(tq, orc, x, xt, gran, axis, g, code, sym, dy=dy)


def test_random_fp8_and_fp4_cases(tq, orc):
    """32 seeded FP8 block cases (block shapes 1 x 16 .. 128 x 128 and odd
    ones, partial edge blocks, all three input types) and 24 FP4 cases
    (NVFP4 / MXFP4, rows 1..300, K a multiple of the block), each through
    quantize, dequantize, STE backward and dequantize backward."""
    from test_parity_fp4 import run_fp4
    from test_parity_fp8 import run_fp8
    rng = np.random.default_rng(1203)
    for case in range(32):
        br = int(rng.choice([1, 1, 1, 2, 4, 8, 16, 32, 64, 128, 3, 5]))
        bc = int(rng.choice([16, 32, 64, 128, 128, 256, 7, 24, 100]))
        rows = int(rng.integers(1, 260))
        cols = int(rng.integers(1, 9)) * int(rng.choice([8, 16, 33, 64, 128]))
        xt = FTS[rng.integers(len(FTS))]
        note("random fp8 case", case)
        x = workloads.normal((rows, cols), float(rng.choice([0.02, 1.0, 300.0])), 7000 + case, xt)
        run_fp8(tq, orc, x, xt, br, bc, dy=workloads.normal((rows, cols), 1.0, 7500 + case, xt))
    for case in range(24):
        kind = ("nvfp4", "mxfp4")[case % 2]
        gs = 16 if kind == "nvfp4" else 32
        rows = int(rng.integers(1, 300))
        k = gs * int(rng.integers(1, 24))
        xt = FTS[rng.integers(len(FTS))]
        note("random fp4 case", case)
        x = workloads.normal((rows, k), float(rng.choice([0.02, 1.0, 50.0])), 8000 + case, xt)
        run_fp4(tq, orc, x, xt, kind, dy=workloads.normal((rows, k), 1.0, 8500 + case, xt))


def test_random_f64_and_mxfp8_cases(tq, orc):
    """24 seeded binary64 cases (every granularity, rank 1-3, integer codes)
    and 16 MXFP8 cases (K a multiple of 32, all three input types)."""
    from test_parity_f64 import run_f64
    from test_parity_mxfp8 import run_mx8
    rng = np.random.default_rng(31)
    for case in range(24):
        gran, shape, axis, g, code, sym, _, _ = _draw(rng)
        note("random f64 case", case)
        x = np.random.default_rng(6000 + case).standard_normal(shape) * float(rng.choice([1e-3, 2.5, 1e5]))
        dy = np.random.default_rng(6500 + case).standard_normal(shape)
        run_f64(tq, orc, x, gran, axis, g, code, sym, dy=dy)
    for case in range(16):
        rows = int(rng.integers(1, 200))
        k = 32 * int(rng.integers(1, 40))
        xt = FTS[rng.integers(len(FTS))]
        note("random mxfp8 case", case)
        x = workloads.normal((rows, k), float(rng.choice([0.02, 1.0, 100.0])), 5000 + case, xt)
        run_mx8(tq, orc, x, xt, dy=workloads.normal((rows, k), 1.0, 5500 + case, xt))


def test_random_fp4_layouts(tq, orc):
    """Seeded random shapes for the GEMM-layout transposes (tiled 256 x 256
    path with ragged tiles, and the generic path) and the transpose-concat
    with padding, against the oracle's numpy layouts."""
    from gpu_util import assert_same, from_dev, to_dev
    rng = np.random.default_rng(77)
    for case in range(16):
        kind = ("nvfp4", "mxfp4")[case % 2]
        gs = 16 if kind == "nvfp4" else 32
        n = int(rng.choice([16, 32, 48, 272, 512, 784, 1000, 1040])) + int(rng.choice([0, 0, 0, 3]))
        k = gs * int(rng.integers(1, 80))
        note("random transpose case", case, n, k, kind)
        x = workloads.normal((n, k), 0.02, 300 + case, "bf16")
        p, b, _ = tq.tq_quant_fp4_block(to_dev(x, "bf16"), kind)
        pt, bt = tq.tq_fp4_transpose_for_gemm(p, b, n, k, gs)
        op, ob = orc.fp4_transpose_for_gemm(from_dev(p), from_dev(b), n, k, gs)
        assert_same(from_dev(pt), op, "packed^T")
        assert_same(from_dev(bt), ob, "scales^T")
    for case in range(8):
        kind = ("nvfp4", "mxfp4")[case % 2]
        gs = 16 if kind == "nvfp4" else 32
        k = gs * int(rng.integers(2, 40))
        ns = [int(rng.choice([0, 16, 48, 256, 272, 300, 512])) for _ in range(int(rng.integers(1, 4)))]
        if sum(ns) == 0:
            ns[0] = 32
        align = int(rng.choice([1, 16, 64, 128, 512]))
        note("random concat case", case, ns, k, kind, align)
        parts = []
        for i, nn in enumerate(ns):
            xx = workloads.normal((nn, k), 0.02, 400 + 10 * case + i, "bf16")
            sgl = torch.tensor([2e-5], dtype=torch.float32, device="cuda") if kind == "nvfp4" else None
            pp, bb, _ = tq.tq_quant_fp4_block(to_dev(xx, "bf16"), kind, global_scale=sgl)
            parts.append((pp, bb))
        pt, bt, stride = tq.tq_fp4_transpose_concat_for_gemm(parts, k, gs, align)
        op, ob, ostride = orc.fp4_transpose_concat([(from_dev(a), from_dev(c)) for a, c in parts], k, gs, align)
        assert stride == ostride
        assert_same(from_dev(pt), op, "packed^T concat")
        assert_same(from_dev(bt), ob, "scales^T concat")
