"""GPU parity on the degenerate scales the fast paths leave to IEEE
division, and on per-tensor sizes at the edge of the partial-maximum
workspace.

- All-tiny groups: every element below about 1e-12, so the group scale is
  under 2^-40 and the kernels take the exact-division branch
  (docs.rs baracuda_kernels::quantize, module overview: scale and STE rule;
  the degenerate reading: a scale of 0 becomes 1).  Rows of tiny and normal
  groups are interleaved so that one launch runs both branches.
- All-subnormal binary32 groups: the symmetric scale RN(amax / qmax) is then
  subnormal and |x / scale| can pass qmax, so the code must clamp
  (190 * 2^-149 with qmax 127 gives scale 2^-149 and x / scale = 190).
- Per-tensor dynamic scale on 8388616 = 1024 * 8192 + 8 elements, where the
  chunk count of the partial maxima reaches its limit of 1024.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import assert_same, from_dev, note, to_dev
from test_parity_fp4 import run_fp4
from test_parity_fp8 import run_fp8
from test_parity_int import run_int_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tq():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import tensor_quantization_amd as t
    return t


def tiny_rows(shape, ft, seed, factor=1e-13, every=2):
    """N(0,1) values with every `every`-th row (or leading-axis slab)
    multiplied by `factor` in binary32 before rounding to the storage type."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(shape).astype(np.float32)
    v[::every] *= np.float32(factor)
    return workloads.to_storage(v, ft)


def subnormal_f32(shape, seed, kmax=400):
    """Integer multiples of 2^-149 in [-kmax, kmax]: every group's amax is
    subnormal, and so is its scale."""
    rng = np.random.default_rng(seed)
    return (rng.integers(-kmax, kmax + 1, shape).astype(np.float32) * np.float32(2.0 ** -149)).astype(np.float32)


TINY_INT = [
    # gran, shape, xt, axis, g, code, sym
    ("token", (8, 4096), "bf16", 0, 0, "s8", True),       # row-group kernel
    ("token", (8, 4096), "f32", 0, 0, "u8", False),
    ("token", (16, 512), "bf16", 0, 0, "s8", True),       # team kernel
    ("token", (6, 7168), "bf16", 0, 0, "s4", True),
    ("token", (6, 100), "f32", 0, 0, "s8", True),         # generic
    ("group", (16, 4096), "bf16", 1, 128, "u4", False),   # g = 128 teams
    ("group", (16, 1024), "f32", 1, 128, "s4", True),
    ("group", (64, 96), "bf16", 0, 32, "u8", False),      # column groups
    ("channel", (128, 64), "f32", 1, 0, "s8", True),
    ("tensor", (4, 256), "f32", 0, 0, "s8", True),
]


@pytest.mark.parametrize("gran,shape,xt,axis,g,code,sym", TINY_INT)
def test_tiny_groups_int(tq, orc, gran, shape, xt, axis, g, code, sym):
    x = tiny_rows(shape, xt, sum(shape) + g)
    if gran == "tensor":                       # one group: make all of it tiny
        x = workloads.to_storage(workloads.normal(shape, 1.0, 3, "f32") * np.float32(1e-13), xt)
    run_int_case(tq, orc, x, xt, gran, axis, g, code, sym, dy=workloads.normal(shape, 1.0, 5, xt))


@pytest.mark.parametrize("shape,block", [((8, 1024), (1, 128)), ((256, 384), (128, 128)), ((6, 40), (2, 8))])
def test_tiny_groups_fp8(tq, orc, shape, block):
    every = 2 if block[0] == 1 else 1
    if every == 1:          # 128 x 128 tiles: make the first block row tiny, the rest normal
        rng = np.random.default_rng(9)
        v = rng.standard_normal(shape).astype(np.float32)
        v[:block[0]] *= np.float32(1e-13)
        x = workloads.to_storage(v, "bf16")
    else:
        x = tiny_rows(shape, "bf16", 7)
    run_fp8(tq, orc, x, "bf16", *block, dy=workloads.normal(shape, 1.0, 8, "bf16"))


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_tiny_blocks_fp4(tq, orc, kind):
    x = tiny_rows((16, 512), "bf16", 11, factor=1e-12)
    dy = workloads.normal((16, 512), 1.0, 12, "bf16")
    run_fp4(tq, orc, x, "bf16", kind, dy=dy)
    if kind == "nvfp4":                        # a tiny static per-tensor scale: every eff tiny
        run_fp4(tq, orc, x, "bf16", kind, static_global=np.float32(1e-30), dy=dy)
        # and an all-tiny tensor with a dynamic one
        xt = workloads.to_storage(workloads.normal((16, 512), 1.0, 13, "f32") * np.float32(1e-30), "bf16")
        run_fp4(tq, orc, xt, "bf16", kind, dy=dy)


SUBNORMAL = [
    ("token", (8, 4096), 0, 0),
    ("token", (16, 512), 0, 0),
    ("token", (4, 7168), 0, 0),
    ("group", (16, 4096), 1, 128),
    ("group", (8, 256), 1, 16),
    ("channel", (64, 64), 1, 0),
    ("channel", (32, 512), 0, 0),
    ("tensor", (64, 256), 0, 0),
    ("tensor", (300, 256), 0, 0),               # two-pass per-tensor path
]


@pytest.mark.parametrize("code", ["s8", "s4"])
@pytest.mark.parametrize("gran,shape,axis,g", SUBNORMAL)
def test_subnormal_groups(tq, orc, gran, shape, axis, g, code):
    x = subnormal_f32(shape, sum(shape) + g)
    run_int_case(tq, orc, x, "f32", gran, axis, g, code, True, dy=workloads.normal(shape, 1.0, 6, "f32"))


def test_subnormal_fake_quant(tq, orc):
    x = subnormal_f32((64, 256), 17).reshape(-1)
    y, s, _ = tq.tq_fake_quant_per_tensor(to_dev(x, "f32"), code="s8")
    oy, os_, _ = orc.fake_quant_per_tensor(x, "f32", code="s8")
    assert_same(from_dev(s).reshape(-1), np.asarray(os_).reshape(-1), "scale")
    assert_same(from_dev(y), oy, "fake quant")


@pytest.mark.parametrize("numel,xt,code,sym", [(8388616, "f32", "s8", True), (8388616, "bf16", "u8", False),
                                               (8388617, "f32", "s8", True)])
def test_per_tensor_partial_limit(tq, orc, numel, xt, code, sym):
    note("per-tensor", numel, xt, code)
    x = workloads.normal((numel,), 1.0, 8, xt)
    run_int_case(tq, orc, x, xt, "tensor", 0, 0, code, sym)
