"""GPU parity of the block-scaled FP8 GEMM against the oracle's binary64
result, within a bound derived from the matrix-core arithmetic.

The E4M3 x E4M3 matrix-core step (128 products per output, one per 128-wide
K block) does not add its products exactly.  Probes of the instruction on
single-wave inputs show: products are taken in groups of eight consecutive
K; inside a group each product is cut toward zero to a multiple of
2^(E - 13), E the group's largest exponent sum ea + eb of the two operands'
exponents (subnormal codes counting as -6); the 16 group sums are then
combined keeping about 24 bits below the largest and the result is
converted toward zero.  The bound used here over-covers each of those steps:
  intra   sum over products that are not multiples of 2^(E + 1 - 13) of that
          granule (zero when the group's exponents lie within 6 of each other)
  cross   17 terms each cut by < 2^-21 of the block's magnitude sum, plus
          2^-23 of it for the final cut
  outer   the block sum times sa * sw and the fused accumulation in binary32:
          (nkb + 2) 2^-24 of the magnitude sum yabs
so |y - y_exact| <= sum_kb |sa sw| intra_kb + (17 2^-21 + 2^-23
+ (nkb + 2) 2^-24) yabs, and a bf16 / f16 output adds its half-ulp rounding.
On random codes over the whole E4M3 range the probes' worst error was a
quarter of this bound."""
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


def _e4m3_tables(orc):
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    with np.errstate(invalid="ignore"):
        val = orc.dequant_fp8_block(codes, 1, 256, np.ones((1, 1), np.float32), "f32").reshape(256).astype(np.float64)
    field = (np.arange(256) >> 3) & 15
    ex = np.where(field == 0, -6, field - 7)
    return val, ex


def intra_bound(orc, qa, sa, qw, sw):
    """sum_kb |sa sw| * (intra-group truncation bound of block kb), per output."""
    val, ex = _e4m3_tables(orc)
    M, K = qa.shape
    N = qw.shape[0]
    nkb = K // 128
    va, ea = val[qa], ex[qa]
    vw, ew = val[qw], ex[qw]
    out = np.zeros((M, N))
    for m in range(M):
        for n0 in range(0, N, 512):
            n1 = min(N, n0 + 512)
            p = va[m][None, :] * vw[n0:n1]                       # [n, K] exact products
            e = (ea[m][None, :] + ew[n0:n1]).astype(np.int32)
            nz = p != 0
            eg = np.where(nz, e, -100).reshape(n1 - n0, K // 8, 8).max(axis=2)
            gran = np.ldexp(1.0, eg + 1 - 13)[:, :, None]
            cut = nz.reshape(n1 - n0, K // 8, 8) & (np.fmod(np.abs(p).reshape(n1 - n0, K // 8, 8), gran) != 0)
            per_group = cut.sum(axis=2) * gran[:, :, 0]
            per_block = per_group.reshape(n1 - n0, nkb, 16).sum(axis=2)   # [n, nkb]
            scale = np.abs(sa[m][None, :].astype(np.float64) * sw[np.arange(n0, n1) // 128].astype(np.float64))
            out[m, n0:n1] = (per_block * scale).sum(axis=1)
    return out


def check(y, ref, yabs, intra, K, yt):
    nkb = K // 128
    bound = intra + (17 * 2.0 ** -21 + 2.0 ** -23 + (nkb + 2) * 2.0 ** -24) * yabs + 1e-30
    if yt == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7)
    elif yt == "f16":
        bound = bound + 2.0 ** -11 * np.abs(ref) * (1 + 2.0 ** -10) + 2.0 ** -25
    err = np.abs(y.astype(np.float64) - ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, ("%d outputs outside the bound; first %s: got %r want %r bound %r"
                           % (len(bad), tuple(bad[0]), y[tuple(bad[0])], ref[tuple(bad[0])], bound[tuple(bad[0])]))
    return float((err / bound).max())


def _as_f32(y, yt):
    yv = from_dev(y)
    if yt != "f32":
        yv = torch.from_numpy(yv.view(np.int16)).view(TORCH[yt]).float().numpy()
    return yv


def _operands(tq, M, N, K, seed):
    x = workloads.normal((M, K), 1.0, seed, "bf16")
    w = workloads.normal((N, K), 0.02, seed + 1, "bf16")
    qa, sa = tq.tq_quant_fp8_block(to_dev(x, "bf16"), 1, 128)
    qw, sw = tq.tq_quant_fp8_block(to_dev(w, "bf16"), 128, 128)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K,yt", [(128, 128, 128, "f32"), (256, 384, 512, "f32"), (128, 256, 1024, "bf16"),
                                      (384, 128, 256, "f16"), (128, 128, 7168, "f32"), (100, 256, 512, "f32"),
                                      (1, 128, 1024, "bf16"), (300, 128, 256, "f32"), (257, 256, 384, "bf16"),
                                      (520, 128, 640, "f32"), (511, 256, 256, "f16"), (1024, 384, 1152, "bf16")])
def test_fp8_block_gemm(tq, orc, M, N, K, yt):
    """Operands from the FP8 quantizers (1 x 128 activations, 128 x 128 weights)."""
    note("fp8 gemm", M, N, K, yt)
    qa, sa, qw, sw = _operands(tq, M, N, K, M + N + K)
    y = tq.tq_fp8_block_gemm(qa, sa, qw, sw, out_dtype=TORCH[yt])
    QA, SA, QW, SW = from_dev(qa), from_dev(sa), from_dev(qw), from_dev(sw)
    ref, yabs = orc.fp8_block_gemm(QA, SA, QW, SW)
    check(_as_f32(y, yt), ref, yabs, intra_bound(orc, QA, SA, QW, SW), K, yt)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 256, 768), (128, 384, 2048)])
def test_fp8_block_gemm_narrow_exponents(tq, orc, M, N, K):
    """Codes with exponents 1 .. 15 only (values 1 .. 15, both signs) and random
    positive scales: no product is cut inside its group, so the bound is the
    binary32 one and checks the scale bookkeeping closely."""
    note("fp8 gemm narrow", M, N, K)
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    def codes(shape):
        return ((rng.integers(7, 11, shape) << 3) | rng.integers(0, 8, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    QA, QW = codes((M, K)), codes((N, K))
    SA = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    SW = rng.uniform(1e-3, 4e-3, (N // 128, K // 128)).astype(np.float32)
    d = lambda a: torch.from_numpy(a).cuda()
    y = tq.tq_fp8_block_gemm(d(QA), d(SA), d(QW), d(SW), out_dtype=torch.float32)
    ref, yabs = orc.fp8_block_gemm(QA, SA, QW, SW)
    intra = intra_bound(orc, QA, SA, QW, SW)
    assert intra.max() == 0.0
    check(from_dev(y), ref, yabs, intra, K, "f32")


@pytest.mark.parametrize("yt", ["f32", "bf16"])
def test_fp8_block_gemm_tiles_agree(tq, yt):
    """M >= 256 runs the 256 x 128 tile, smaller M the 128 x 128 one; both
    take the same block sums and binary32 scale-and-add steps in the same
    order, so the first rows of a 300-row product equal, bit for bit, the
    product of those rows alone."""
    note("fp8 gemm tiles agree", yt)
    qa, sa, qw, sw = _operands(tq, 300, 256, 896, 77)
    big = from_dev(tq.tq_fp8_block_gemm(qa, sa, qw, sw, out_dtype=TORCH[yt]))
    small = from_dev(tq.tq_fp8_block_gemm(qa[:200].contiguous(), sa[:200].contiguous(), qw, sw, out_dtype=TORCH[yt]))
    assert_same(big[:200], small, "rows 0..199")


def test_fp8_block_gemm_full_size_sampled(tq, orc):
    """The c4 operands: activations bf16 [4096, 7168] (1 x 128) times weights
    bf16 [7168, 7168] (128 x 128), bf16 out as timed: rows sampled for the
    oracle, all columns."""
    note("fp8 gemm full size")
    x = workloads.make_input("c4_fp8_act_1x128")
    w = workloads.make_input("c4_fp8_weight_128x128")
    qa, sa = tq.tq_quant_fp8_block(to_dev(x, "bf16"), 1, 128)
    qw, sw = tq.tq_quant_fp8_block(to_dev(w, "bf16"), 128, 128)
    y = tq.tq_fp8_block_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16)
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 256, 2049, 4095])
    QA, SA, QW, SW = from_dev(qa)[rows], from_dev(sa)[rows], from_dev(qw), from_dev(sw)
    ref, yabs = orc.fp8_block_gemm(QA, SA, QW, SW)
    check(_as_f32(y, "bf16")[rows], ref, yabs, intra_bound(orc, QA, SA, QW, SW), 7168, "bf16")


def test_fp8_block_gemm_shapes(tq):
    qa = torch.zeros((100, 128), dtype=torch.uint8, device="cuda")
    sa = torch.ones((100, 1), dtype=torch.float32, device="cuda")
    qw = torch.zeros((100, 128), dtype=torch.uint8, device="cuda")
    sw = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError):                       # N = 100: weights come in 128-row tiles
        tq.tq_fp8_block_gemm(qa, sa, qw, sw)
    qw = torch.zeros((128, 128), dtype=torch.uint8, device="cuda")
    y = tq.tq_fp8_block_gemm(qa[:0], sa[:0], qw, sw)
    assert y.numel() == 0
    y = tq.tq_fp8_block_gemm(torch.zeros((128, 0), dtype=torch.uint8, device="cuda"),
                             torch.zeros((128, 0), dtype=torch.float32, device="cuda"),
                             torch.zeros((128, 0), dtype=torch.uint8, device="cuda"),
                             torch.zeros((1, 0), dtype=torch.float32, device="cuda"), out_dtype=torch.float32)
    assert y.shape == (128, 128) and bool((y == 0).all())


# ------------------------------------------------------- W8A8 quantized linear
def _w8a8_operands(tq, x, xt, w, wt):
    qx, sx, _ = tq.tq_quant_per_token(to_dev(x, xt))
    qw, sw, _ = tq.tq_quant_per_token(to_dev(w, wt))
    return qx, sx, qw, sw


def _i8(t):
    return from_dev(t).view(np.int8)


@pytest.mark.parametrize("M,N,K,yt", [(128, 128, 128, "f32"), (256, 384, 512, "bf16"), (100, 256, 1024, "f16"),
                                      (1, 128, 4096, "bf16"), (300, 128, 256, "f32"), (128, 128, 7168, "f32"),
                                      (300, 512, 768, "bf16"), (1, 256, 128, "f32")])
def test_w8a8_linear(tq, orc, M, N, K, yt):
    """Bit-exact against the oracle: per-token s8 activations (1% outlier
    columns x20, as in the activation workload) times per-channel s8 weights."""
    note("w8a8", M, N, K, yt)
    x = workloads.normal_with_outlier_columns((M, K), 1.0, M + K, "bf16", 0.01, 20.0, K)
    w = workloads.normal((N, K), 0.02, N + K, "f16")
    qx, sx, qw, sw = _w8a8_operands(tq, x, "bf16", w, "f16")
    y = tq.tq_w8a8_linear(qx, sx, qw, sw, out_dtype=TORCH[yt])
    assert_same(from_dev(y), orc.w8a8_linear(_i8(qx), from_dev(sx), _i8(qw), from_dev(sw), yt), "y")


@pytest.mark.parametrize("M,N", [(128, 128), (128, 256), (300, 128), (300, 256)])
def test_w8a8_linear_extreme_codes(tq, orc, M, N):
    """All codes at -128 / 127 / 0 patterns: the largest integer sums, and
    sums past 2^24 that the conversion to binary32 must round to nearest
    (every tile kernel: M >= 256 takes the 256-row tile)."""
    note("w8a8 extreme", M, N)
    K = 4096
    rng = np.random.default_rng(7)
    QX = rng.choice(np.array([-128, 127, 0, -127], np.int8), (M, K))
    QW = rng.choice(np.array([-128, 127, 1], np.int8), (N, K))
    QX[0, :] = -128
    QW[0, :] = -128                                       # acc = 2^26 exactly
    SX = rng.uniform(1e-4, 1e-2, M).astype(np.float32)
    SW = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    d = lambda a: torch.from_numpy(a).cuda()
    y = tq.tq_w8a8_linear(d(QX), d(SX), d(QW), d(SW), out_dtype=torch.float32)
    assert_same(from_dev(y), orc.w8a8_linear(QX, SX, QW, SW, "f32"), "y")


def test_w8a8_linear_full_size_sampled(tq, orc):
    """The activation workload bf16 [8192, 4096] (per-token s8) times the
    weight workload f16 [11008, 4096] (per-channel s8), bf16 out as timed:
    rows sampled for the oracle, all columns."""
    note("w8a8 full size")
    x = workloads.make_input("c2_per_token_s8")
    w = workloads.make_input("c3_per_group_u4_g128")
    qx, sx, qw, sw = _w8a8_operands(tq, x, "bf16", w, "f16")
    y = tq.tq_w8a8_linear(qx, sx, qw, sw, out_dtype=torch.bfloat16)
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 256, 4097, 8191])
    ref = orc.w8a8_linear(_i8(qx)[rows], from_dev(sx)[rows], _i8(qw), from_dev(sw), "bf16")
    assert_same(from_dev(y)[rows], ref, "y")


def test_w8a8_linear_shapes(tq):
    z8 = lambda r, c: torch.zeros((r, c), dtype=torch.int8, device="cuda")
    ones = lambda n: torch.ones(n, dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError):
        tq.tq_w8a8_linear(z8(4, 128), ones(4), z8(100, 128), ones(100))      # N % 128
    y = tq.tq_w8a8_linear(z8(3, 0), ones(3), z8(128, 0), ones(128), out_dtype=torch.float32)
    assert y.shape == (3, 128) and bool((y == 0).all())


# ------------------------------------------------------ FP4 weight-only linear
def check_fp4(y, ref, yabs, K, yt):
    """Bound from the bf16 matrix-core arithmetic (probed on single-wave
    inputs): a step aligns its 32 exact bf16 x bf16 products and its
    accumulator input to the largest of them, keeps bits down to 2^(E - 24)
    and rounds the sum to nearest.  A 64-wide block is two chained steps from
    zero: <= (32 + 1 + 33 + 1) 2^-24 of the block's magnitude sum, taken
    four times over here; each block sum is then added in binary32
    (2^-24 of the running magnitude) and the NVFP4 per-tensor scale applied
    once (2^-24)."""
    nkb = K // 64
    bound = (4 * 67 + nkb + 1) * 2.0 ** -24 * yabs + 1e-30
    if yt == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref) * (1 + 2.0 ** -7)
    elif yt == "f16":
        bound = bound + 2.0 ** -11 * np.abs(ref) * (1 + 2.0 ** -10) + 2.0 ** -25
    err = np.abs(y.astype(np.float64) - ref)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, ("%d outputs outside the bound; first %s: got %r want %r bound %r"
                           % (len(bad), tuple(bad[0]), y[tuple(bad[0])], ref[tuple(bad[0])], bound[tuple(bad[0])]))
    return float((err / bound).max())


def _fp4_weight(tq, w, kind):
    packed, bs, sg = tq.tq_quant_fp4_block(to_dev(w, "bf16"), kind)
    return packed, bs, sg


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("M,N,K,yt", [(128, 128, 64, "f32"), (256, 256, 512, "f32"), (100, 384, 1024, "bf16"),
                                      (1, 128, 4096, "f16"), (300, 128, 4096, "f32"), (128, 128, 192, "f32"),
                                      (200, 256, 320, "bf16"), (257, 256, 320, "bf16"), (520, 128, 640, "f16"),
                                      (1024, 256, 1024, "bf16")])
def test_fp4_linear(tq, orc, kind, M, N, K, yt):
    """bf16 activations (1% outlier columns x20) times an FP4 weight quantized
    on the GPU from bf16 ~N(0, 0.02).  The kernel walks K in pairs of 64-wide
    blocks; K = 64, 192 and 320 leave one block after the pairs."""
    note("fp4 linear", kind, M, N, K, yt)
    x = workloads.normal_with_outlier_columns((M, K), 1.0, M + K + 1, "bf16", 0.01, 20.0, K)
    w = workloads.normal((N, K), 0.02, N + K + 2, "bf16")
    packed, bs, sg = _fp4_weight(tq, w, kind)
    y = tq.tq_fp4_linear(to_dev(x, "bf16"), packed, bs, sg, kind, out_dtype=TORCH[yt])
    ref, yabs = orc.fp4_linear(x, from_dev(packed), from_dev(bs), from_dev(sg) if sg is not None else 1.0, kind)
    check_fp4(_as_f32(y, yt), ref, yabs, K, yt)


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_fp4_linear_tiles_agree(tq, kind):
    """M >= 256 runs the 256 x 128 tile, smaller M the 128 x 128 one: the
    same block sums and binary32 adds in the same order, so the first rows
    of a 300-row product equal, bit for bit, the product of those rows alone."""
    note("fp4 linear tiles agree", kind)
    x = to_dev(workloads.normal((300, 960), 1.0, 91, "bf16"), "bf16")
    packed, bs, sg = _fp4_weight(tq, workloads.normal((256, 960), 0.02, 92, "bf16"), kind)
    big = from_dev(tq.tq_fp4_linear(x, packed, bs, sg, kind, out_dtype=torch.float32))
    small = from_dev(tq.tq_fp4_linear(x[:200].contiguous(), packed, bs, sg, kind, out_dtype=torch.float32))
    assert_same(big[:200], small, "rows 0..199")


def test_fp4_linear_full_size_sampled(tq, orc):
    """The bf16 [8192, 4096] activations times the NVFP4 weight workload
    [14336, 4096], bf16 out as timed: rows sampled for the oracle."""
    note("fp4 linear full size")
    x = workloads.make_input("c2_per_token_s8")
    w = workloads.make_input("c5_fp4_weight")
    packed, bs, sg = _fp4_weight(tq, w, "nvfp4")
    y = tq.tq_fp4_linear(to_dev(x, "bf16"), packed, bs, sg, "nvfp4", out_dtype=torch.bfloat16)
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 256, 4097, 8191])
    ref, yabs = orc.fp4_linear(x[rows], from_dev(packed), from_dev(bs), from_dev(sg), "nvfp4")
    check_fp4(_as_f32(y, "bf16")[rows], ref, yabs, 4096, "bf16")


def test_fp4_linear_shapes(tq):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros((100, 32), dtype=torch.uint8, device="cuda")
    b = torch.zeros((100, 4), dtype=torch.uint8, device="cuda")
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError):                       # N % 128
        tq.tq_fp4_linear(x, p, b, g, "nvfp4")
    p128 = torch.zeros((128, 32), dtype=torch.uint8, device="cuda")
    b128 = torch.zeros((128, 4), dtype=torch.uint8, device="cuda")
    with pytest.raises(tq.TQError):                       # f16 activations
        tq.tq_fp4_linear(x.half(), p128, b128, g, "nvfp4")
    y = tq.tq_fp4_linear(x[:, :0], torch.zeros((128, 0), dtype=torch.uint8, device="cuda"),
                         torch.zeros((128, 0), dtype=torch.uint8, device="cuda"), g, "nvfp4", out_dtype=torch.float32)
    assert y.shape == (4, 128) and bool((y == 0).all())


def test_random_gemm_shapes(tq, orc):
    """Seeded random (M, N, K, output type) for the three GEMMs: M any size
    (ragged last tile), N a multiple of 128 (so both W8A8 tiles run), K a
    multiple of 128 (64 for the FP4 linear); the same checks as above."""
    rng = np.random.default_rng(4096)
    for case in range(10):
        M = int(rng.integers(1, 400))
        N = 128 * int(rng.integers(1, 5))
        K = 128 * int(rng.integers(1, 9))
        yt = ("f32", "bf16", "f16")[int(rng.integers(3))]
        note("random gemm case", case, M, N, K, yt)
        qa, sa, qw, sw = _operands(tq, M, N, K, 300 + case)
        y = tq.tq_fp8_block_gemm(qa, sa, qw, sw, out_dtype=TORCH[yt])
        QA, SA, QW, SW = from_dev(qa), from_dev(sa), from_dev(qw), from_dev(sw)
        ref, yabs = orc.fp8_block_gemm(QA, SA, QW, SW)
        check(_as_f32(y, yt), ref, yabs, intra_bound(orc, QA, SA, QW, SW), K, yt)

        x = workloads.normal_with_outlier_columns((M, K), 1.0, 400 + case, "bf16", 0.01, 20.0, K)
        w = workloads.normal((N, K), 0.02, 500 + case, "f16")
        qx, sx, qw8, sw8 = _w8a8_operands(tq, x, "bf16", w, "f16")
        y = tq.tq_w8a8_linear(qx, sx, qw8, sw8, out_dtype=TORCH[yt])
        assert_same(from_dev(y), orc.w8a8_linear(_i8(qx), from_dev(sx), _i8(qw8), from_dev(sw8), yt), "w8a8 y")

        kind = ("nvfp4", "mxfp4")[case % 2]
        K4 = 64 * int(rng.integers(1, 17))
        x4 = workloads.normal_with_outlier_columns((M, K4), 1.0, 600 + case, "bf16", 0.01, 20.0, K4)
        w4 = workloads.normal((N, K4), 0.02, 700 + case, "bf16")
        packed, bs, sg = _fp4_weight(tq, w4, kind)
        y = tq.tq_fp4_linear(to_dev(x4, "bf16"), packed, bs, sg, kind, out_dtype=TORCH[yt])
        ref, yabs = orc.fp4_linear(x4, from_dev(packed), from_dev(bs), from_dev(sg) if sg is not None else 1.0, kind)
        check_fp4(_as_f32(y, yt), ref, yabs, K4, yt)
