"""Pins of the oracle's floating-point-code backward rules and the FP4
dequantization (CPU only).

Rules (docs.rs baracuda_kernels::quantize, module overview and module list;
smile.llm.quant Fp8BlockGemm; metrale QuantizedWeight, fields):
  quantize backward    dx = (dy / scale) * 1[lo < val(q) < hi], q recomputed
                       from the saved input and the saved scale;
                       E4M3: lo, hi = -448, 448; E2M1: -6, 6;
                       NVFP4 scale = val(sb) * s_g, MXFP4 scale = 2^(sb - 127)
  dequantize backward  dq = dy * scale
  FP4 dequantize       y = val(q) * (val(sb) * s_g)   (MXFP4: val(q) * 2^(sb-127))

The expected values here never come from the oracle: codes are found by
exhaustive nearest-value search over the format's value list
(tests/bruteforce.py), the binary32 quotient and products by numpy float32,
the storage types are widened by numpy (f16) and torch (bf16) and narrowed by
the same libraries, and the saturation edges are the hand-worked rows of
tests/golden/ste_saturation_edges.txt.
"""
import os

import numpy as np
import pytest
import torch

import bruteforce as bf
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ independent helpers
def widen_ref(x, xt):
    """Storage -> float32 by library casts (not the oracle's decoders)."""
    if xt == "f32":
        return np.asarray(x, np.float32)
    if xt == "f16":
        return np.asarray(x, np.uint16).view(np.float16).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).numpy()


def narrow_ref(v, xt):
    return workloads.to_storage(np.asarray(v, np.float32), xt)


def e4m3_table():
    mags = bf.e4m3_magnitudes()
    dec = np.full(256, np.nan, np.float64)
    dec[:127], dec[128:255] = mags, -mags
    dec[128] = -0.0
    return dec


def e2m1_table():
    mags = bf.e2m1_magnitudes()
    dec = np.concatenate([mags, -mags])
    dec[8] = -0.0
    return dec


def e4m3_code(v):
    return bf.nearest_code(np.asarray(v, np.float32), bf.e4m3_magnitudes(), 0x80)


def e2m1_code(v):
    return bf.nearest_code(np.asarray(v, np.float32), bf.e2m1_magnitudes(), 0x8)


def div32(a, b):
    with np.errstate(all="ignore"):
        return (np.asarray(a, np.float32) / np.asarray(b, np.float32)).astype(np.float32)


def mul32(a, b):
    with np.errstate(all="ignore"):
        return (np.asarray(a, np.float32) * np.asarray(b, np.float32)).astype(np.float32)


def read_edges():
    rows = []
    with open(os.path.join(GOLDEN, "ste_saturation_edges.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            fmt, tbits, _tdec, code, val, mask = line.split()
            rows.append((fmt, np.uint32(int(tbits, 16)).view(np.float32), int(code, 16), float(val), int(mask)))
    return rows


EDGES = read_edges()


# ------------------------------------------------------------ bf16 widening
def test_bf16_widen_all_patterns(orc):
    """Every bf16 pattern widens to the binary32 value torch's cast gives
    (NaN patterns: NaN of the same sign)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    want = widen_ref(h, "bf16")
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (np.signbit(got[nan]) == np.signbit(want[nan])).all()
    assert (got[~nan].view(np.uint32) == want[~nan].view(np.uint32)).all()
    assert np.array_equal(orc.widen(h, "bf16")[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ------------------------------------------------------------ golden saturation edges
def test_golden_edges_are_consistent():
    """The hand-worked rows agree with the exhaustive nearest-value search
    and with the mask rule on the decoded value (a check of the fixture)."""
    for fmt, t, code, val, mask in EDGES:
        c = (e4m3_code([t]) if fmt == "e4m3" else e2m1_code([t]))[0]
        dec = (e4m3_table() if fmt == "e4m3" else e2m1_table())[c]
        hi = 448.0 if fmt == "e4m3" else 6.0
        assert c == code, (fmt, t)
        assert dec == val and np.signbit(dec) == np.signbit(val), (fmt, t)
        assert int(-hi < dec < hi) == mask, (fmt, t)


def test_golden_edges_reject_unrounded_mask():
    """The fixture separates the rule from the plausible misreading that
    masks on the unrounded quotient (|x / scale| < bound): at least one row
    per format disagrees with it."""
    for fmt in ("e2m1", "e4m3"):
        hi = 448.0 if fmt == "e4m3" else 6.0
        rows = [r for r in EDGES if r[0] == fmt]
        assert any(int(abs(float(t)) < hi) != mask for _, t, _, _, mask in rows), fmt


@pytest.mark.parametrize("scale_exp", [0, -3, 5])
def test_fp8_block_ste_golden_edges(orc, scale_exp):
    """Each E4M3 edge row placed in a 1 x 8 block with a static scale 2^e
    (x = t * 2^e exactly): dx = dy / 2^e where the row's mask is 1, else a
    zero with the sign of dy / scale."""
    rows = [r for r in EDGES if r[0] == "e4m3"]
    n = len(rows)
    cols = 8
    s = np.float32(2.0 ** scale_exp)
    x = np.zeros((n, cols), np.float32)
    for i, (_, t, _, _, _) in enumerate(rows):
        x[i, :] = np.float32(t) * s
    dy = np.array([[(-1.0) ** (i + j) * (1.5 + j) for j in range(cols)] for i in range(n)], np.float32)
    scale = np.full((n, 1), s, np.float32)
    dx = orc.quant_fp8_block_backward(x, "f32", 1, cols, scale, dy)
    for i, (_, t, _, _, mask) in enumerate(rows):
        want = div32(dy[i], s) * np.float32(mask)
        assert (dx[i].view(np.uint32) == want.view(np.uint32)).all(), (t, dx[i], want)


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_fp4_ste_golden_edges(orc, kind):
    """Each E2M1 edge row in its own FP4 block.  NVFP4 with s_g = 1 and block
    scale 0x38 (1.0), or s_g = 2^-4 with 0x48 (4.0) so eff = 0.25; MXFP4 with
    sb = 127 - 2 (eff = 0.25).  x = t * eff exactly."""
    rows = [r for r in EDGES if r[0] == "e2m1"]
    gs = 16 if kind == "nvfp4" else 32
    n = len(rows)
    if kind == "nvfp4":
        sg, sb = np.float32(2.0 ** -4), 0x48
        eff = np.float32(4.0 * 2.0 ** -4)
    else:
        sg, sb = np.float32(1.0), 125
        eff = np.float32(0.25)
    x = np.zeros((n, gs), np.float32)
    for i, (_, t, _, _, _) in enumerate(rows):
        x[i, :] = np.float32(t) * eff
    dy = np.array([[(-1.0) ** j * (0.75 + j) for j in range(gs)] for _ in range(n)], np.float32)
    bscale = np.full((n, 1), sb, np.uint8)
    dx = orc.quant_fp4_block_backward(x, "f32", bscale, sg, kind, dy)
    for i, (_, t, _, _, mask) in enumerate(rows):
        want = div32(dy[i], eff) * np.float32(mask)
        assert (dx[i].view(np.uint32) == want.view(np.uint32)).all(), (t, dx[i], want)
    # the same with NVFP4 s_g = 1, block scale 1.0: x = t itself
    if kind == "nvfp4":
        x1 = np.repeat(np.array([[r[1]] for r in rows], np.float32), gs, axis=1)
        dx1 = orc.quant_fp4_block_backward(x1, "f32", np.full((n, 1), 0x38, np.uint8), np.float32(1.0), kind, dy)
        masks = np.array([r[4] for r in rows], np.float32)[:, None]
        assert (dx1.view(np.uint32) == (dy * masks).view(np.uint32)).all()


# ------------------------------------------------------------ FP8 blocks: brute force
def _fp8_blocks(shape, br, bc):
    nbr, nbc = -(-shape[0] // br), -(-shape[1] // bc)
    rr = np.minimum(np.arange(shape[0]) // br, nbr - 1)
    cc = np.minimum(np.arange(shape[1]) // bc, nbc - 1)
    return rr[:, None] * nbc + cc[None, :], (nbr, nbc)


@pytest.mark.parametrize("shape,block,xt,shrink", [
    ((4, 256), (1, 128), "bf16", 1.0),
    ((256, 256), (128, 128), "f32", 1.3),      # scales below amax / 448: many codes saturate
    ((6, 20), (4, 8), "f16", 1.1),             # partial blocks on both edges
    ((3, 128), (1, 128), "bf16", 0.7),
])
def test_fp8_block_backward_bruteforce(orc, shape, block, xt, shrink):
    """STE and dequantize backward of the FP8 block family against a
    brute-force derivation: scale per block from the block amax (or that
    scale shrunk, so that elements reach and pass 448), codes by nearest
    E4M3 search, mask on the decoded value."""
    br, bc = block
    x = workloads.normal(shape, 2.0, 91, xt)
    dy = workloads.normal(shape, 1.0, 92, xt)
    xv, dyv = widen_ref(x, xt), widen_ref(dy, xt)
    bid, (nbr, nbc) = _fp8_blocks(shape, br, bc)
    amax = np.zeros(nbr * nbc, np.float32)
    np.maximum.at(amax, bid.ravel(), np.abs(xv).ravel())
    s = div32(amax, np.float32(448.0 * shrink))
    s = np.where(s == 0, np.float32(1), s).astype(np.float32)
    scale = s.reshape(nbr, nbc)
    se = s[bid]
    t = div32(xv, se)
    val = e4m3_table()[e4m3_code(t)]
    mask = ((val > -448) & (val < 448)).astype(np.float32)
    if shrink > 1:
        assert (mask == 0).sum() > 0 and (mask == 1).sum() > 0
    want_dx = narrow_ref(mul32(div32(dyv, se), mask), xt)
    dx = orc.quant_fp8_block_backward(x, xt, br, bc, scale, dy)
    assert (dx == want_dx).all()
    want_dq = narrow_ref(mul32(dyv, se), xt)
    dq = orc.dequant_fp8_block_backward(dy, xt, br, bc, scale)
    assert (dq == want_dq).all()


def test_fp8_block_ste_signed_zero_gradients(orc):
    """Masked elements give a zero with the sign of dy / scale (a product,
    not a select); -0 inputs are inside the range."""
    x = np.array([[448.0, -448.0, 0.0, -0.0, 500.0, -500.0, 1.0, -1.0]], np.float32)
    dy = np.array([[-2.0, 2.0, -0.0, 3.0, 1.0, -1.0, -4.0, 5.0]], np.float32)
    dx = orc.quant_fp8_block_backward(x, "f32", 1, 8, np.ones((1, 1), np.float32), dy)
    want = np.array([[-0.0, 0.0, -0.0, 3.0, 0.0, -0.0, -4.0, 5.0]], np.float32)
    assert (dx.view(np.uint32) == want.view(np.uint32)).all()


# ------------------------------------------------------------ FP4: brute force
def _fp4_eff(kind, sb, sg):
    if kind == "nvfp4":
        return mul32(e4m3_table()[sb].astype(np.float32), sg)
    return np.ldexp(np.float32(1), sb.astype(np.int32) - 127).astype(np.float32)


def _random_scale_bytes(kind, n, rng):
    if kind == "nvfp4":
        b = rng.integers(0, 127, n)                 # finite non-negative E4M3 (0x00 .. 0x7e)
    else:
        b = rng.integers(0, 255, n)                 # every finite E8M0 byte
    return b.astype(np.uint8)


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("yt", ["f32", "bf16", "f16"])
def test_fp4_dequant_exact(orc, kind, yt):
    """val(q) * eff with eff = val(sb) * s_g (one binary32 product each),
    then one rounding to the output type: random codes, every kind of block
    scale byte (zero, subnormal, normal, the largest), several s_g."""
    rng = np.random.default_rng(17)
    gs = 16 if kind == "nvfp4" else 32
    rows, k = 24, 8 * gs
    packed = rng.integers(0, 256, (rows, k // 2)).astype(np.uint8)
    sb = _random_scale_bytes(kind, rows * (k // gs), rng).reshape(rows, k // gs)
    if kind == "nvfp4":
        sb[0, :] = [0x00, 0x01, 0x07, 0x08, 0x38, 0x7e, 0x40, 0x30][: k // gs]
    else:
        sb[0, :] = [0, 1, 126, 127, 128, 254, 100, 150][: k // gs]
    codes = np.stack([packed & 0xF, packed >> 4], -1).reshape(rows, k)
    dec = e2m1_table().astype(np.float32)[codes]
    for sg in ([np.float32(1.0)] if kind == "mxfp4" else
               [np.float32(1.0), np.float32(0.02 / 2688 * 3.7), np.float32(2.0 ** -130), np.float32(1e30)]):
        eff = np.repeat(_fp4_eff(kind, sb, sg), gs, axis=1)
        want = narrow_ref(mul32(dec, eff), yt)
        got = orc.dequant_fp4_block(packed, sb, sg, kind, yt)
        assert (got == want).all(), (kind, yt, sg)


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("xt", ["bf16", "f32"])
def test_fp4_backward_bruteforce(orc, kind, xt):
    """STE and dequantize backward of the FP4 blocks on random inputs, with
    the block scales the quantizer picks and with random ones (which push
    many elements past 6, and many to 0)."""
    rng = np.random.default_rng(23)
    gs = 16 if kind == "nvfp4" else 32
    rows, k = 12, 4 * gs
    x = workloads.normal((rows, k), 0.02, 31, xt)
    dy = workloads.normal((rows, k), 1.0, 32, xt)
    xv, dyv = widen_ref(x, xt), widen_ref(dy, xt)
    _, sb_q, sg_q = orc.quant_fp4_block(x, xt, kind)
    sg_q = np.float32(np.asarray(sg_q).ravel()[0])
    sb_r = _random_scale_bytes(kind, rows * (k // gs), rng).reshape(rows, k // gs)
    if kind == "nvfp4":
        sb_r = np.where(sb_r < 0x20, sb_r + 0x20, sb_r).astype(np.uint8)   # keep eff above the bf16 range floor
        cases = [(sb_q, sg_q), (sb_r, np.float32(0.02 / 2688)), (sb_r, np.float32(1.0))]
    else:
        sb_r = (np.uint8(115) + (sb_r % 12)).astype(np.uint8)                # 2^-12 .. 2^-1
        cases = [(sb_q, np.float32(1.0)), (sb_r, np.float32(1.0))]
    saw_masked = False
    for sb, sg in cases:
        eff = np.repeat(_fp4_eff(kind, sb, sg), gs, axis=1)
        t = div32(xv, eff)
        val = e2m1_table()[e2m1_code(t)]
        mask = ((val > -6) & (val < 6)).astype(np.float32)
        saw_masked |= bool((mask == 0).any())
        want_dx = narrow_ref(mul32(div32(dyv, eff), mask), xt)
        dx = orc.quant_fp4_block_backward(x, xt, sb, sg, kind, dy)
        assert (dx == want_dx).all(), (kind, xt, sg)
        want_dq = narrow_ref(mul32(dyv, eff), xt)
        dq = orc.dequant_fp4_block_backward(dy, xt, sb, sg, kind)
        assert (dq == want_dq).all(), (kind, xt, sg)
    assert saw_masked


def test_fp4_ste_quantizer_scales_mask_each_block_max(orc):
    """With the quantizer's own NVFP4 scales, the element at each block's
    |x| max decodes to +-6 (amax / eff lies in [5.65, 6.4]) and so gets a
    zero gradient -- the FP analogue of amax -> +-qmax."""
    x = workloads.normal((16, 64), 0.02, 41, "bf16")
    dy = workloads.normal((16, 64), 1.0, 42, "bf16")
    _, sb, sg = orc.quant_fp4_block(x, "bf16", "nvfp4")
    dx = widen_ref(orc.quant_fp4_block_backward(x, "bf16", sb, np.asarray(sg).ravel()[0], "nvfp4", dy), "bf16")
    xv = widen_ref(x, "bf16").reshape(16, 4, 16)
    j = np.abs(xv).argmax(axis=2)
    picked = np.take_along_axis(dx.reshape(16, 4, 16), j[..., None], axis=2)
    assert (picked == 0).all()
