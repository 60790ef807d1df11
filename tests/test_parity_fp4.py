"""GPU parity of the FP4 E2M1 family (NVFP4 with dynamic or static per-tensor
scale, MXFP4; quantize, dequantize, STE, dequantize backward, transpose to
GEMM layout) against the oracle, bit for bit, plus a dense check of the E2M1
conversion."""
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


def run_fp4(tq, orc, x, xt, kind, static_global=None, dy=None):
    note("fp4 case", x.shape, xt, kind, "static" if static_global is not None else "dynamic")
    xd = to_dev(x, xt)
    sgd = None if static_global is None else torch.tensor([static_global], dtype=torch.float32, device="cuda")
    p, b, g = tq.tq_quant_fp4_block(xd, kind, global_scale=sgd)
    op, ob, og = orc.quant_fp4_block(x, xt, kind, static_global=static_global)
    assert_same(from_dev(p), op, "packed")
    assert_same(from_dev(b), ob, "block scales")
    if kind == "nvfp4":
        assert_same(from_dev(g), og, "global scale")
    for yt in {xt, "f32"}:
        y = tq.tq_dequant_fp4_block(p, b, g, kind, out_dtype=TORCH[yt])
        assert_same(from_dev(y), orc.dequant_fp4_block(op, ob, og[0], kind, yt), "dequant->" + yt)
    if dy is None:
        dy = workloads.normal(x.shape, 1.0, 99, xt)
    dyd = to_dev(dy, xt)
    dx = tq.tq_quant_fp4_block_backward(xd, dyd, b, g, kind)
    assert_same(from_dev(dx), orc.quant_fp4_block_backward(x, xt, ob, og[0], kind, dy), "ste")
    dq = tq.tq_dequant_fp4_block_backward(dyd, b, g, kind)
    assert_same(from_dev(dq), orc.dequant_fp4_block_backward(dy, xt, ob, og[0], kind), "dq")
    return p, b


@pytest.mark.parametrize("shape,xt,kind", [
    ((64, 4096), "bf16", "nvfp4"), ((64, 4096), "bf16", "mxfp4"),
    ((37, 160), "f16", "nvfp4"), ((37, 160), "f32", "mxfp4"),
    ((3, 32), "bf16", "nvfp4"), ((1, 96), "f16", "mxfp4"),
    ((300, 48), "f32", "nvfp4"),
])
def test_fp4(tq, orc, shape, xt, kind):
    x = workloads.normal(shape, 0.02, shape[0] + shape[1], xt)
    run_fp4(tq, orc, x, xt, kind)


def test_nvfp4_static_global(tq, orc):
    x = workloads.normal((48, 512), 0.02, 5, "bf16")
    run_fp4(tq, orc, x, "bf16", "nvfp4", static_global=np.float32(3.1e-5))


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("xt", ["bf16", "f32"])
def test_fp4_degenerate_values(tq, orc, kind, xt):
    x = nasty((32, 256), xt, 21)
    x[0, :64] = 0
    x[1, 32:64] = workloads.to_storage(np.full(32, 1e-6, np.float32), xt)
    run_fp4(tq, orc, x, xt, kind, dy=nasty((32, 256), xt, 22))


def test_e2m1_conversion_dense(tq, orc):
    """MXFP4 blocks whose max |x| lies in [4, 8) get E8M0 byte 127 (scale 1),
    so their codes are the E2M1 encodings of the inputs: a dense sweep of
    binary32 values in [2^-8, 7.99] (every 7th pattern), both signs."""
    lo, hi = np.float32(2.0 ** -8).view(np.uint32), np.float32(7.99).view(np.uint32)
    v = np.arange(lo, hi, 7, dtype=np.uint32).view(np.float32)
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float32)])
    n = (v.size + 30) // 31 * 31
    v = np.concatenate([v, np.zeros(n - v.size, np.float32)]).reshape(-1, 31)
    x = np.concatenate([np.full((v.shape[0], 1), 4.0, np.float32), v], axis=1)
    p, b, _ = tq.tq_quant_fp4_block(to_dev(x, "f32"), "mxfp4")
    assert (from_dev(b) == 127).all()
    codes = orc.enc_e2m1(x)
    assert_same(from_dev(p), codes[:, 0::2] | (codes[:, 1::2] << 4), "E2M1 codes")


def test_transpose_for_gemm(tq, orc):
    # tiled path with whole tiles, tiled path with ragged 256 x 256 tiles in
    # both directions, generic path (rows not a multiple of 16)
    for (n, k, kind) in [(14336 // 7, 4096, "nvfp4"), (256, 1024, "mxfp4"), (784, 1056, "nvfp4"),
                         (528, 2080, "mxfp4"), (40, 96, "nvfp4"), (24, 64, "mxfp4")]:
        gs = 16 if kind == "nvfp4" else 32
        x = workloads.normal((n, k), 0.02, n + k, "bf16")
        p, b, _ = tq.tq_quant_fp4_block(to_dev(x, "bf16"), kind)
        pt, bt = tq.tq_fp4_transpose_for_gemm(p, b, n, k, gs)
        op, ob = orc.fp4_transpose_for_gemm(from_dev(p), from_dev(b), n, k, gs)
        assert_same(from_dev(pt), op, "packed^T %s" % ((n, k),))
        assert_same(from_dev(bt), ob, "scales^T %s" % ((n, k),))


def _quant_parts(tq, ns, k, kind, seed0):
    parts = []
    for i, n in enumerate(ns):
        x = workloads.normal((n, k), 0.02, seed0 + i, "bf16")
        sg = torch.tensor([2e-5], dtype=torch.float32, device="cuda") if kind == "nvfp4" else None
        p, b, _ = tq.tq_quant_fp4_block(to_dev(x, "bf16"), kind, global_scale=sg)
        parts.append((p, b))
    return parts


@pytest.mark.parametrize("ns,k,kind,align", [
    ([2048, 512, 512], 4096, "nvfp4", 1),       # fused QKV-like: tiled path, no pad
    ([256, 128], 1024, "mxfp4", 512),           # tiled path, 128 pad columns
    ([272, 48], 544, "nvfp4", 1),               # tiled path, ragged tiles, part offset inside a tile
    ([1001], 256, "nvfp4", 16),                 # odd N: generic path, 7 pad columns
    ([40, 24, 33], 96, "nvfp4", 64),            # ragged parts
    ([0, 48, 0, 16], 64, "mxfp4", 1),           # empty parts
])
def test_transpose_concat_for_gemm(tq, orc, ns, k, kind, align):
    note("transpose_concat", ns, k, kind, align)
    gs = 16 if kind == "nvfp4" else 32
    parts = _quant_parts(tq, ns, k, kind, 700 + k)
    pt, bt, stride = tq.tq_fp4_transpose_concat_for_gemm(parts, k, gs, align)
    host = [(from_dev(p), from_dev(b)) for p, b in parts]
    op, ob, ostride = orc.fp4_transpose_concat(host, k, gs, align)
    assert stride == ostride
    assert_same(from_dev(pt), op, "packed^T concat")
    assert_same(from_dev(bt), ob, "scales^T concat")
    # codes only
    pt2, bt2, _ = tq.tq_fp4_transpose_concat_for_gemm([(p, None) for p, _ in parts], k, gs, align)
    assert bt2 is None
    assert_same(from_dev(pt2), op, "packed^T concat, codes only")


def test_transpose_concat_rejects_empty_list(tq):
    with pytest.raises(tq.TQError):
        tq.tq_fp4_transpose_concat_for_gemm([], 64, 16)


def test_transpose_concat_full_size(tq, orc):
    """[14336, 4096] gate and up projections fused into one [2048, 28672]
    NVFP4 GEMM operand (tiled path), every byte against the oracle."""
    note("transpose_concat full size")
    w = workloads.make_input("c5_fp4_weight")
    p, b, g = tq.tq_quant_fp4_block(to_dev(w, "bf16"), "nvfp4")
    up = (torch.flip(p, [0]).contiguous(), torch.flip(b, [0]).contiguous())   # a second weight, same shape
    pt, bt, stride = tq.tq_fp4_transpose_concat_for_gemm([(p, b), up], 4096, 16, 128)
    assert stride == 28672
    parts = [(from_dev(p), from_dev(b)), (from_dev(up[0]), from_dev(up[1]))]
    opt, obt, ostride = orc.fp4_transpose_concat(parts, 4096, 16, 128)
    assert ostride == stride
    assert_same(from_dev(pt), opt, "packed^T")
    assert_same(from_dev(bt), obt, "scales^T")


@pytest.mark.parametrize("n1,n2,k", [(96, 40, 4096), (3, 5, 48), (7, 0, 32)])
def test_concat_rows(tq, orc, n1, n2, k):
    """16-byte units (aligned rows), 8-byte and 1-byte units (rows of 24 code
    bytes and 3 scale bytes put the second part at unaligned offsets)."""
    note("concat_rows", n1, n2, k)
    parts = _quant_parts(tq, [n1, max(n2, 1)], k, "nvfp4", 800)
    if n2 == 0:
        parts[1] = (parts[1][0][:0], parts[1][1][:0])
    (p1, b1), (p2, b2) = parts
    g = np.float32(2e-5)
    po, bo = tq.tq_fp4_concat_rows(p1, b1, g, p2, b2, g, k)
    op, ob = orc.fp4_concat_rows(from_dev(p1), from_dev(b1), g, from_dev(p2), from_dev(b2), g, k)
    assert_same(from_dev(po), op, "rows packed")
    assert_same(from_dev(bo), ob, "rows scales")
    with pytest.raises(tq.TQError):
        tq.tq_fp4_concat_rows(p1, b1, g, p2, b2, np.nextafter(g, np.float32(1)), k)
    with pytest.raises(tq.TQError):
        tq.tq_fp4_concat_rows(p1, b1, 0.0, p2, b2, -0.0, k)


@pytest.mark.parametrize("shape,kind,scale_x", [((64, 4096), "nvfp4", 1.0), ((64, 4096), "mxfp4", 1.0),
                                                ((37, 160), "nvfp4", 50.0), ((3, 96), "mxfp4", 1e4),
                                                ((1, 16), "nvfp4", 1.0)])
def test_predequant_to_fp8(tq, orc, shape, kind, scale_x):
    note("predequant_to_fp8", shape, kind, scale_x)
    x = workloads.normal(shape, 0.02 * scale_x, shape[0] * 7 + shape[1], "f32")
    x[0, :16] = 0.0
    p, b, g = tq.tq_quant_fp4_block(to_dev(x, "f32"), kind)
    gh = float(from_dev(g)[0]) if kind == "nvfp4" else 1.0
    out = tq.tq_fp4_predequant_to_fp8(p, b, gh, kind)
    assert_same(from_dev(out), orc.fp4_predequant_to_fp8(from_dev(p), from_dev(b), np.float32(gh), kind), "e4m3")


def test_predequant_degenerate_scales(tq, orc):
    """Every E4M3 block-scale byte with each of a few per-tensor scales
    (products that saturate, fall in the E4M3 subnormals or underflow),
    every E2M1 code pair."""
    note("predequant degenerate")
    codes = np.arange(256, dtype=np.uint8)
    packed = np.tile(codes[None, :], (256, 1))          # row r: every code pair; k = 512
    bscale = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 512 // 16, axis=1)
    bscale[(bscale & 0x7F) == 0x7F] = 0x38                                  # no NaN scales
    for sg in (1.0, 2.0 ** -20, 3.0e3, 7.1e-3):
        out = tq.tq_fp4_predequant_to_fp8(to_dev(packed), to_dev(bscale), sg, "nvfp4")
        assert_same(from_dev(out), orc.fp4_predequant_to_fp8(packed, bscale, np.float32(sg), "nvfp4"),
                    "e4m3 sg=%g" % sg)
    mx = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 512 // 32, axis=1)
    mx[mx == 255] = 127                                                       # 0xFF is the E8M0 NaN
    out = tq.tq_fp4_predequant_to_fp8(to_dev(packed), to_dev(mx), 1.0, "mxfp4")
    assert_same(from_dev(out), orc.fp4_predequant_to_fp8(packed, mx, np.float32(1.0), "mxfp4"), "e4m3 mx")


def test_predequant_full_size(tq, orc):
    note("predequant full size")
    w = workloads.make_input("c5_fp4_weight")
    for kind in ("nvfp4", "mxfp4"):
        p, b, g = tq.tq_quant_fp4_block(to_dev(w, "bf16"), kind)
        gh = float(from_dev(g)[0]) if kind == "nvfp4" else 1.0
        out = from_dev(tq.tq_fp4_predequant_to_fp8(p, b, gh, kind))
        assert_same(out, orc.fp4_predequant_to_fp8(from_dev(p), from_dev(b), np.float32(gh), kind), kind + " e4m3")
