"""Pins of the oracle's FP4 layout follow-ons (metrale QuantizedWeight:
transpose_concat_for_gemm / _gs / _padded, concat_rows, predequant_to_fp8).

The concatenations are byte moves: they are pinned to numpy's own transpose
and concatenate.  The FP8 expansion is pinned to an independent computation:
E2M1 values from the golden table times the E4M3 block-scale value (from the
format's enumeration) times the per-tensor scale in numpy float32, then a
brute-force nearest E4M3 code.
"""
import numpy as np
import pytest

import bruteforce as bf
import workloads


def _fp4_weight(orc, rows, k, seed, kind="nvfp4", sg=None):
    x = workloads.normal((rows, k), 0.02, seed, "bf16")
    return orc.quant_fp4_block(x, "bf16", kind, static_global=sg)


def _numpy_concat_t(parts, align):
    cat_p = np.concatenate([p.T for p, _ in parts], axis=1)
    cat_s = np.concatenate([s.T for _, s in parts], axis=1)
    total = cat_p.shape[1]
    stride = -(-total // align) * align
    return (np.pad(cat_p, ((0, 0), (0, stride - total))), np.pad(cat_s, ((0, 0), (0, stride - total))), stride)


@pytest.mark.parametrize("ns,align,gs", [([48], 1, 16), ([40, 8, 24], 1, 16), ([33, 7, 1], 16, 16),
                                         ([5, 11], 64, 32), ([0, 17], 8, 16)])
def test_transpose_concat_matches_numpy(orc, ns, align, gs):
    k = 128
    kind = "nvfp4" if gs == 16 else "mxfp4"
    parts = []
    for i, n in enumerate(ns):
        p, s, _ = _fp4_weight(orc, n, k, 1000 + i, kind, sg=np.float32(1e-4) if kind == "nvfp4" else None)
        parts.append((p, s))
    pt, st, stride = orc.fp4_transpose_concat(parts, k, gs, align)
    wp, ws, wstride = _numpy_concat_t(parts, align)
    assert stride == wstride and stride % align == 0 and stride - sum(ns) < align
    assert np.array_equal(pt, wp) and np.array_equal(st, ws)
    assert not pt[:, sum(ns):].any() and not st[:, sum(ns):].any()


def test_transpose_concat_single_part_is_plain_transpose(orc):
    p, s, _ = _fp4_weight(orc, 40, 64, 7, sg=np.float32(1e-3))
    pt, st, stride = orc.fp4_transpose_concat([(p, s)], 64, 16)
    tp, ts = orc.fp4_transpose_for_gemm(p, s, 40, 64, 16)
    assert stride == 40 and np.array_equal(pt, tp) and np.array_equal(st, ts)


def test_transpose_concat_empty_list_rejected(orc):
    with pytest.raises(ValueError):
        orc.fp4_transpose_concat([], 64, 16)


def test_concat_rows_matches_numpy(orc):
    sg = np.float32(3e-4)
    p1, s1, g1 = _fp4_weight(orc, 24, 96, 11, sg=sg)
    p2, s2, g2 = _fp4_weight(orc, 9, 96, 12, sg=sg)
    po, so = orc.fp4_concat_rows(p1, s1, g1[0], p2, s2, g2[0], 96)
    assert np.array_equal(po, np.concatenate([p1, p2])) and np.array_equal(so, np.concatenate([s1, s2]))


@pytest.mark.parametrize("g1,g2", [(1e-3, np.nextafter(np.float32(1e-3), np.float32(1))), (0.0, -0.0)])
def test_concat_rows_needs_bit_identical_scales(orc, g1, g2):
    p, s, _ = _fp4_weight(orc, 4, 32, 13, sg=np.float32(1e-3))
    with pytest.raises(ValueError):
        orc.fp4_concat_rows(p, s, np.float32(g1), p, s, np.float32(g2), 32)


def _predequant_brute(packed, bscale, sg, kind):
    e2m1 = bf.e2m1_magnitudes()
    e4m3 = bf.e4m3_magnitudes()
    rows, kb = packed.shape
    k = kb * 2
    lo, hi = packed & 0xF, packed >> 4
    codes = np.empty((rows, k), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    vals = np.where(codes & 8, -1.0, 1.0) * e2m1[codes & 7]
    gs = 16 if kind == "nvfp4" else 32
    sb = np.repeat(bscale, gs, axis=1)
    if kind == "nvfp4":
        sbv = np.where(sb & 0x80, -1.0, 1.0) * e4m3[sb & 0x7F]
        eff = (sbv.astype(np.float32) * np.float32(sg)).astype(np.float32)
    else:
        eff = np.ldexp(np.float32(1), sb.astype(np.int32) - 127).astype(np.float32)
    prod = (vals.astype(np.float32) * eff).astype(np.float32)
    return bf.nearest_code(prod, e4m3, 0x80)


@pytest.mark.parametrize("kind,sg,scale_x", [("nvfp4", None, 1.0), ("nvfp4", 2e-2, 1.0), ("nvfp4", 1.0, 50.0),
                                             ("mxfp4", None, 1.0), ("mxfp4", None, 1e4)])
def test_predequant_to_fp8_matches_brute_force(orc, kind, sg, scale_x):
    x = workloads.normal((16, 256), 0.02 * scale_x, 21, "f32")
    x[0, :16] = 0.0                                   # an all-zero block
    x[1, :32] *= 1e-6                                  # products below the E4M3 subnormal range
    p, s, g = orc.quant_fp4_block(x, "f32", kind, static_global=None if sg is None else np.float32(sg))
    gsc = g[0] if kind == "nvfp4" else 1.0
    got = orc.fp4_predequant_to_fp8(p, s, gsc, kind)
    want = _predequant_brute(p, s, gsc, kind)
    assert np.array_equal(got, want)


def test_predequant_saturates_and_keeps_zero_sign(orc):
    # codes: +6 (0x7), -0 (0x8), +0.5 (0x1), -6 (0xF); one NVFP4 block with sb = 448 (0x7E)
    packed = np.array([[0x87, 0xF1] + [0] * 6], np.uint8)
    bscale = np.array([[0x7E]], np.uint8)
    got = orc.fp4_predequant_to_fp8(packed, bscale, np.float32(1.0), "nvfp4")
    assert got[0, 0] == 0x7E and got[0, 1] == 0x80 and got[0, 3] == 0xFE     # 6*448 saturates to +-448
    assert got[0, 2] == 0x76                                                   # 0.5 * 448 = 224 = 1.75 * 2^7
    assert not got[0, 4:].any()
