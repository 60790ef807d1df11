"""Pins of the oracle's scalar format conversions (CPU only).

Each test compares the oracle with something other than itself: the OCP
value definitions (golden fixtures), exhaustive nearest-value search, or a
library cast (numpy's float16, torch's bfloat16 / float8_e4m3fn).
"""
import numpy as np
import pytest
import torch

import bruteforce as bf


def test_e2m1_table_matches_ocp_values(orc):
    codes, vals = bf.read_table("e2m1_values.txt")
    tab = orc.dec_e2m1_table()
    assert len(codes) == 16
    for c, v in zip(codes, vals):
        assert tab[c] == v and np.signbit(tab[c]) == np.signbit(v), hex(c)


def test_e4m3_table_matches_ocp_points_and_torch(orc):
    tab = orc.dec_e4m3_table()
    codes, vals = bf.read_table("e4m3_points.txt")
    for c, v in zip(codes, vals):
        if np.isnan(v):
            assert np.isnan(tab[c]), hex(c)
        else:
            assert tab[c] == v and np.signbit(tab[c]) == np.signbit(v), hex(c)
    # all 256 codes against torch's float8_e4m3fn decode (a library routine)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    same = (tab == ref) | (np.isnan(tab) & np.isnan(ref))
    assert same.all()
    # against the structural enumeration: 127 finite non-negative values
    mags = bf.e4m3_magnitudes()
    assert len(mags) == 127 and mags[-1] == 448.0 and mags[1] == 2.0 ** -9
    assert (tab[:127] == mags).all() and (tab[128:255] == -mags).all()


def _dense_f32(lo_exp, hi_exp, stride, seed=0):
    """Every stride-th binary32 pattern with exponent in [lo_exp, hi_exp),
    both signs, plus zeros."""
    lo = (lo_exp + 127) << 23
    hi = (hi_exp + 127) << 23
    bits = np.arange(lo, hi, stride, dtype=np.uint32)
    v = bits.view(np.float32)
    return np.concatenate([v, -v, np.array([0.0, -0.0], np.float32)])


def _midpoints(mags):
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert (mid.astype(np.float64) == (mags[:-1] + mags[1:]) / 2).all()   # exact
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    m = np.concatenate([mid, up, dn, mags.astype(np.float32)])
    return np.concatenate([m, -m])


def test_e4m3_encode_is_nearest_even_saturating(orc):
    mags = bf.e4m3_magnitudes()
    v = np.concatenate([
        _dense_f32(-20, 10, 97),                       # dense sweep, subnormal to saturated
        _midpoints(mags),                              # every tie and its neighbours
        np.array([448, 449, 464, 465, 1e6, 3e38, 2 ** -10, -2 ** -10, 2 ** -11, 1e-30, -1e-30],
                 np.float32),
    ])
    got = orc.enc_e4m3(v)
    want = bf.nearest_code(v, mags, 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_e4m3_encode_matches_torch_cast_in_range(orc):
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(2_000_000).astype(np.float32) * np.float32(40.0))
    v = np.concatenate([v, _midpoints(bf.e4m3_magnitudes())])
    v = v[np.abs(v) <= 448]                            # torch does not saturate above 448
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (orc.enc_e4m3(v) == ref).all()


def test_e2m1_encode_ties_and_nearest(orc):
    # hand-derived ties of the E2M1 grid (ties go to the even mantissa)
    ties = {0.25: 0x0, 0.75: 0x2, 1.25: 0x2, 1.75: 0x4, 2.5: 0x4, 3.5: 0x6, 5.0: 0x6, 7.0: 0x7}
    for v, c in ties.items():
        assert orc.enc_e2m1(np.array([v], np.float32))[0] == c, v
        assert orc.enc_e2m1(np.array([-v], np.float32))[0] == c | 0x8, -v
    mags = bf.e2m1_magnitudes()
    v = np.concatenate([_dense_f32(-8, 5, 13), _midpoints(mags),
                        np.array([-1e-20, 1e-20, -0.0, 6.0, 6.5, 100.0], np.float32)])
    got = orc.enc_e2m1(v)
    want = bf.nearest_code(v, mags, 0x8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_e8m0_mx_scale_puts_amax_in_top_e2m1_binade(orc):
    # OCP MX v1.0 shared scale for E2M1 elements: X = 2^(floor(log2 amax) - 2),
    # i.e. the unique power of two with amax / X in [4, 8).
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(200_000).astype(np.float32)) * np.float32(
        2.0) ** rng.integers(-100, 100, 200_000).astype(np.float32)
    amax = amax[(amax > 2.0 ** -120) & (amax < 2.0 ** 120)]
    b = orc.enc_e8m0_mx(amax)
    X = np.array([orc.dec_e8m0(int(c)) for c in b[:2000]], np.float64)
    r = amax[:2000].astype(np.float64) / X
    assert ((r >= 4) & (r < 8)).all()
    # vectorised on all: 2^(b-127) via ldexp
    r = amax.astype(np.float64) / np.ldexp(1.0, b.astype(np.int64) - 127)
    assert ((r >= 4) & (r < 8)).all()
    # clamped ends and the all-zero block (reading: scale 1.0, byte 127)
    assert orc.enc_e8m0_mx(np.array([0.0], np.float32))[0] == 127
    assert orc.enc_e8m0_mx(np.array([1e-45], np.float32))[0] == 0
    # largest finite binary32 has floor(log2) = 127 -> byte 127 - 2 + 127 = 252
    assert orc.enc_e8m0_mx(np.array([3.4e38], np.float32))[0] == 252
    assert orc.dec_e8m0(127) == 1.0 and orc.dec_e8m0(0) == np.float32(2.0 ** -127)


def _random_finite_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def test_bf16_narrowing_matches_torch(orc):
    v = _random_finite_f32(3_000_000, 11)
    # ties: patterns whose low 16 bits are exactly 0x8000, and neighbours
    rng = np.random.default_rng(12)
    hi = rng.integers(0, 0x7f7f, 100_000, dtype=np.uint32) << 16
    ties = np.concatenate([hi | 0x8000, hi | 0x7fff, hi | 0x8001]).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.array([3.4e38, -3.4e38, 0.0, -0.0, 1e-45], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (orc.narrow_bf16(v) == ref).all()


def test_f16_narrowing_matches_numpy(orc):
    v = np.concatenate([_random_finite_f32(1_000_000, 13),
                        (np.random.default_rng(14).standard_normal(2_000_000) * 0.02).astype(np.float32),
                        _dense_f32(-26, 17, 301),
                        np.array([65504, 65519.99, 65520, 65536, 2 ** -24, 2 ** -25, 3 * 2 ** -26],
                                 np.float32)])
    # numpy's float32 -> float16 cast rounds to nearest even, with subnormals
    # and overflow to inf
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert (orc.narrow_f16(v) == ref).all()


def test_f16_widening_all_patterns(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
