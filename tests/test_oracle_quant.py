"""Pins of the oracle's quantize / dequantize / STE definitions (CPU only).

The oracle is compared with: hand-worked examples (golden fixtures), a
brute-force re-derivation on tiny tensors (groups enumerated by explicit
index loops, roundings by exhaustive nearest-value search, binary32 steps by
numpy float32), closed-form properties (amax maps to +-qmax, round-trip error
within half a step, the STE mask), granularity identities, row independence
and re-quantization idempotence.

Readings that no outside source fixes -- the asymmetric zero-point formula,
the NVFP4 two-level scale bits, MX clipping, degenerate groups -- are pinned
here by the brute-force re-derivation and by closed forms and special cases;
no printed value exists to compare them with.
"""
import itertools
import zlib

import numpy as np
import pytest
import torch

import bruteforce as bf
import workloads

RNG = np.random.default_rng(1234)


def _values(x, xt):
    import oracle
    return oracle.widen(x, xt).astype(np.float32)


def _narrow(v32, ft):
    return workloads.to_storage(np.asarray(v32, np.float32), ft)


def _unpack(q, code, shape):
    q = np.asarray(q, np.uint8)
    if code in ("s4", "u4"):
        lo = (q & 0xF).astype(np.int32)
        hi = (q >> 4).astype(np.int32)
        v = np.stack([lo, hi], axis=-1).reshape(shape)
        if code == "s4":
            v = np.where(v >= 8, v - 16, v)
        return v
    v = q.reshape(shape).astype(np.int32)
    return np.where(v >= 128, v - 256, v) if code == "s8" else v


# ------------------------------------------------------------ brute force
def bf_groups(shape, gran, axis=0, g=0):
    """List of (group id, flat element indices) by explicit index loops."""
    idx = np.arange(int(np.prod(shape))).reshape(shape)
    groups = []
    if gran == "tensor":
        return [(0, idx.ravel())]
    if gran == "token":
        m = idx.reshape(-1, shape[-1])
        return [(r, m[r]) for r in range(m.shape[0])]
    if gran == "channel":
        return [(a, np.take(idx, a, axis=axis).ravel()) for a in range(shape[axis])]
    sshape = list(shape)
    sshape[axis] //= g
    for sidx in itertools.product(*[range(n) for n in sshape]):
        members = []
        for j in range(g):
            full = list(sidx)
            full[axis] = sidx[axis] * g + j
            members.append(idx[tuple(full)])
        groups.append((int(np.ravel_multi_index(sidx, sshape)), np.array(members)))
    return groups


def bf_nearest_int(v, qmin, qmax, zp):
    """Vectorised exhaustive nearest code on the grid c - zp, ties to even."""
    v = np.asarray(v, np.float64)[:, None]
    c = np.arange(qmin, qmax + 1)[None, :]
    d = np.abs(v - (c - zp))
    best = d.min(axis=1, keepdims=True)
    cand = (d == best)
    even = ((c - zp) % 2 == 0)
    pick = np.where(cand.sum(axis=1) > 1, np.argmax(cand & even, axis=1), np.argmax(cand, axis=1))
    return (qmin + pick).astype(np.int32)


def bf_quant_int(xv, shape, gran, axis, g, qmin, qmax, symmetric):
    groups = bf_groups(shape, gran, axis, g)
    n = len(groups)
    scale = np.zeros(n, np.float32)
    zp = np.zeros(n, np.int32)
    codes = np.zeros(xv.size, np.int32)
    flat = xv.ravel()
    for gid, members in groups:
        vals = flat[members]
        if symmetric:
            s = bf.div32(np.max(np.abs(vals)), qmax)
            if s == 0:
                s = np.float32(1)
            z = 0
        else:
            mn = np.float32(min(vals.min(), 0))
            mx = np.float32(max(vals.max(), 0))
            s = bf.div32(np.float32(mx - mn), qmax - qmin)
            if s == 0:
                s = np.float32(1)
            # zero-point reading: the code of real 0 (see module docstring)
            z = int(np.clip(qmin - round(float(bf.div32(mn, s))), qmin, qmax))
        scale[gid], zp[gid] = s, z
        codes[members] = bf_nearest_int(bf.div32(vals, s), qmin, qmax, z)
    return codes.reshape(shape), scale, zp


# ------------------------------------------------------------ golden
def _read_worked(name):
    rows = []
    with open(bf.GOLDEN + "/" + name) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_worked_per_token_s8(orc):
    x, s, q, dy, dx = _read_worked("per_token_s8_worked.txt")
    x = np.array([float(v) for v in x], np.float32)[None, :]
    dy = np.array([float(v) for v in dy], np.float32)[None, :]
    qo, so, _ = orc.quant_int(x, "f32", "token", code="s8", symmetric=True)
    assert so[0] == float(s[0])
    assert (_unpack(qo, "s8", x.shape)[0] == [int(v) for v in q]).all()
    dxo = orc.quant_int_backward(x, "f32", "token", code="s8", symmetric=True, scale=so, dy=dy)
    want = np.array([float(v) for v in dx], np.float32)
    assert (dxo[0].view(np.uint32) == want.view(np.uint32)).all()   # signed zeros too


def test_worked_u4_packing(orc):
    (packed,) = _read_worked("u4_pack_worked.txt")
    x = np.arange(16, dtype=np.float32)[None, :]
    q, s, z = orc.quant_int(x, "f32", "group", axis=1, group_size=16, code="u4", symmetric=False)
    assert s[0, 0] == 1.0 and z[0, 0] == 0
    assert [int(b) for b in q[0]] == [int(v, 16) for v in packed]


# ------------------------------------------------------------ brute force
CASES_INT = [
    # shape, xt, gran, axis, g, code, symmetric
    ((3, 16), "f32", "token", 0, 0, "s8", True),
    ((2, 8), "bf16", "token", 0, 0, "s8", True),
    ((2, 24), "f16", "token", 0, 0, "u8", False),
    ((4, 6), "f32", "tensor", 0, 0, "s8", True),
    ((4, 6), "f32", "tensor", 0, 0, "s8", False),
    ((5, 4), "bf16", "channel", 0, 0, "s8", True),
    ((5, 4), "f16", "channel", 1, 0, "u8", False),
    ((2, 3, 4), "f32", "channel", 1, 0, "s4", True),
    ((3, 256), "f16", "group", 1, 128, "u4", False),
    ((2, 32), "bf16", "group", 1, 8, "s4", False),
    ((8, 4), "f32", "group", 0, 4, "u4", False),
    ((2, 4, 6), "f16", "group", 1, 2, "s8", True),
    ((1, 128), "f32", "group", 1, 128, "s8", False),
]


@pytest.mark.parametrize("shape,xt,gran,axis,g,code,sym", CASES_INT)
def test_bruteforce_integer(orc, shape, xt, gran, axis, g, code, sym):
    seed = zlib.crc32(repr((shape, xt, gran, axis, g, code, sym)).encode())
    x = workloads.normal(shape, 1.0, seed, xt)
    qmin, qmax = orc.default_q_range(code, sym)
    q, s, z = orc.quant_int(x, xt, gran, axis=axis, group_size=g, code=code, symmetric=sym)
    xv = _values(x, xt)
    codes, bs, bz = bf_quant_int(xv, shape, gran, axis, g, qmin, qmax, sym)
    assert (s.ravel().view(np.uint32) == bs.view(np.uint32)).all()
    if not sym:
        assert (z.ravel().astype(np.int32) == bz).all()
    assert (_unpack(q, code, shape) == codes).all()
    # dequant: (q - zp) * scale, rounded once to the output type
    y = orc.dequant_int(q, code, shape, gran, axis, g, s, z, yt=xt)
    groups = bf_groups(shape, gran, axis, g)
    yref = np.zeros(int(np.prod(shape)), np.float32)
    for gid, m in groups:
        yref[m] = bf.mul32(np.float32(codes.ravel()[m] - bz[gid]), bs[gid])
    assert (y.ravel() == _narrow(yref, xt)).all()
    # STE: dx = (dy / scale) * 1[qmin < q < qmax]
    dy = workloads.normal(shape, 1.0, seed + 1, xt)
    dx = orc.quant_int_backward(x, xt, gran, axis, g, code=code, qmin=qmin, qmax=qmax,
                                symmetric=sym, scale=s, zp=z, dy=dy)
    dyv = _values(dy, xt).ravel()
    dref = np.zeros_like(yref)
    for gid, m in groups:
        c = codes.ravel()[m]
        mask = ((c > qmin) & (c < qmax)).astype(np.float32)
        dref[m] = bf.mul32(bf.div32(dyv[m], bs[gid]), mask)
    assert (dx.ravel() == _narrow(dref, xt)).all()
    # dequant backward: dq = dy * scale
    dq = orc.dequant_int_backward(dy, xt, gran, axis, g, s)
    dqref = np.zeros_like(yref)
    for gid, m in groups:
        dqref[m] = bf.mul32(dyv[m], bs[gid])
    assert (dq.ravel() == _narrow(dqref, xt)).all()


@pytest.mark.parametrize("shape,block,xt", [((4, 256), (1, 128), "bf16"), ((256, 256), (128, 128), "f32"),
                                            ((6, 16), (2, 8), "f16")])
def test_bruteforce_fp8_block(orc, shape, block, xt):
    x = workloads.normal(shape, 3.0, 77, xt)
    q, s = orc.quant_fp8_block(x, xt, *block)
    xv = _values(x, xt)
    mags = bf.e4m3_magnitudes()
    br, bc = block
    for i in range(shape[0] // br):
        for j in range(shape[1] // bc):
            blk = xv[i * br:(i + 1) * br, j * bc:(j + 1) * bc]
            sc = bf.div32(np.abs(blk).max(), 448)
            sc = np.float32(1) if sc == 0 else sc
            assert s[i, j].view(np.uint32) == sc.view(np.uint32)
            want = bf.nearest_code(bf.div32(blk, sc), mags, 0x80)
            assert (q[i * br:(i + 1) * br, j * bc:(j + 1) * bc] == want).all()
    y = orc.dequant_fp8_block(q, br, bc, s, xt)
    tab = {c: v for c, v in zip(*bf.read_table("e4m3_points.txt"))}
    vals = np.concatenate([mags, -mags]).astype(np.float32)
    dec = np.zeros(256, np.float32)
    dec[:127] = mags
    dec[128:255] = -mags
    assert all(dec[c] == v for c, v in tab.items() if not np.isnan(v))
    srep = np.repeat(np.repeat(s, br, 0), bc, 1)
    assert (y == _narrow(bf.mul32(dec[q], srep), xt)).all()


def _bf_mx_byte(amax):
    if amax == 0:
        return 127
    for b in range(0, 255):
        r = float(amax) / 2.0 ** (b - 127)
        if 4 <= r < 8:
            return b
    return 0 if float(amax) < 4 * 2.0 ** -127 else 254


@pytest.mark.parametrize("kind", ["nvfp4", "mxfp4"])
def test_bruteforce_fp4(orc, kind):
    rows, k = 3, 64
    x = workloads.normal((rows, k), 0.02, 99, "bf16")
    xv = _values(x, "bf16")
    xv_sm = xv.copy()
    packed, bs, sg = orc.quant_fp4_block(x, "bf16", kind)
    gs = 16 if kind == "nvfp4" else 32
    m2 = bf.e2m1_magnitudes()
    m8 = bf.e4m3_magnitudes()
    dec8 = np.zeros(256, np.float32)
    dec8[:127] = m8
    if kind == "nvfp4":
        g = bf.div32(np.abs(xv).max(), 2688)
        assert sg[0].view(np.uint32) == g.view(np.uint32)
    codes = np.zeros((rows, k), np.uint8)
    for r in range(rows):
        for b in range(k // gs):
            blk = xv_sm[r, b * gs:(b + 1) * gs]
            amax = np.abs(blk).max()
            if kind == "nvfp4":
                sb = bf.nearest_code(np.array([bf.div32(amax, bf.mul32(6, sg[0]))]), m8, 0x80)[0]
                sb = 0x38 if dec8[sb] == 0 else sb
                eff = bf.mul32(dec8[sb], sg[0])
            else:
                sb = _bf_mx_byte(amax)
                eff = np.float32(2.0 ** (sb - 127))
            assert bs[r, b] == sb
            codes[r, b * gs:(b + 1) * gs] = bf.nearest_code(bf.div32(blk, eff), m2, 0x8)
    assert (packed == (codes[:, 0::2] | (codes[:, 1::2] << 4))).all()


# ------------------------------------------------------------ properties
def test_amax_maps_to_qmax(orc):
    x = workloads.normal((64, 512), 1.0, 5, "bf16")
    xv = _values(x, "bf16")
    q, s, _ = orc.quant_int(x, "bf16", "token", code="s8", symmetric=True)
    codes = _unpack(q, "s8", x.shape)
    am = np.argmax(np.abs(xv), axis=1)
    assert (np.abs(codes[np.arange(64), am]) == 127).all()
    q8, s8 = orc.quant_fp8_block(x, "bf16", 1, 128)
    for r in range(64):
        for b in range(4):
            blk = xv[r, b * 128:(b + 1) * 128]
            j = np.argmax(np.abs(blk))
            assert q8[r, b * 128 + j] & 0x7F == 0x7E
    p, bs, sg = orc.quant_fp4_block(x, "bf16", "nvfp4")
    codes4 = np.stack([p & 0xF, p >> 4], -1).reshape(64, 512)
    for r in range(64):
        for b in range(32):
            blk = xv[r, b * 16:(b + 1) * 16]
            if np.abs(blk).max() == 0:
                continue
            j = np.argmax(np.abs(blk))
            assert codes4[r, b * 16 + j] & 0x7 == 0x7        # +-6
    # asymmetric: the minimum maps to qmin exactly
    qa, sa, za = orc.quant_int(x, "bf16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    ca = _unpack(qa, "u4", x.shape)
    for r in range(64):
        for b in range(4):
            blk = xv[r, b * 128:(b + 1) * 128]
            if blk.min() < 0:
                assert ca[r, b * 128 + np.argmin(blk)] == 0


def test_round_trip_within_half_step(orc):
    x = workloads.make_input("c2_per_token_s8", rows=32)
    xv = _values(x, "bf16")
    q, s, _ = orc.quant_int(x, "bf16", "token", code="s8", symmetric=True)
    y = orc.dequant_int(q, "s8", x.shape, "token", scale=s, yt="f32")
    # half a step, plus the binary32 rounding of x / scale (and of the
    # product) that can move a value onto a tie: |x| * 2^-23 covers both
    err = np.abs(y.astype(np.float64) - xv)
    bound = s.astype(np.float64)[:, None] / 2 + np.abs(xv) * 2.0 ** -23
    assert (err <= bound).all()
    w = workloads.make_input("c3_per_group_u4_g128", rows=16)
    wv = _values(w, "f16")
    q, s, z = orc.quant_int(w, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    y = orc.dequant_int(q, "u4", w.shape, "group", 1, 128, s, z, yt="f32")
    srep = np.repeat(s, 128, axis=1).astype(np.float64)
    assert (np.abs(y - wv) <= srep / 2 + (np.abs(wv) + srep * 16) * 2.0 ** -23).all()
    # FP8: half the local grid spacing times the scale
    q8, s8 = orc.quant_fp8_block(x, "bf16", 1, 128)
    y8 = orc.dequant_fp8_block(q8, 1, 128, s8, "f32")
    sr = np.repeat(s8, 128, axis=1).astype(np.float64)
    v = np.abs(xv / sr)
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    half_step = 2.0 ** (e - 3) / 2 * sr
    assert (np.abs(y8 - xv) <= half_step + np.abs(xv) * 2.0 ** -23).all()


def test_ste_mask_on_c1(orc):
    x = workloads.make_input("c1_per_tensor_s8")
    dy = workloads.make_dy("c1_per_tensor_s8")
    q, s, _ = orc.quant_int(x, "f32", "tensor", code="s8", symmetric=True)
    codes = _unpack(q, "s8", x.shape)
    dx = orc.quant_int_backward(x, "f32", "tensor", code="s8", symmetric=True, scale=s, dy=dy)
    at_edge = np.abs(codes) == 127
    assert at_edge.sum() >= 1
    assert (dx[at_edge] == 0).all()
    assert (np.signbit(dx[at_edge]) == np.signbit(dy[at_edge])).all()
    inner = ~at_edge
    assert (dx[inner] == bf.div32(dy[inner], s[0])).all()


def test_granularity_identities(orc):
    x = workloads.normal((6, 40), 1.0, 21, "bf16")
    qa, sa, _ = orc.quant_int(x, "bf16", "token", code="s8")
    qb, sb, _ = orc.quant_int(x, "bf16", "channel", axis=0, code="s8")
    qc, sc, _ = orc.quant_int(x, "bf16", "group", axis=1, group_size=40, code="s8")
    assert (qa == qb).all() and (qa == qc).all()
    assert (sa == sb).all() and (sa == sc.ravel()).all()
    # per-channel along axis 1 == per-group along axis 0 with g = rows
    qd, sd, zd = orc.quant_int(x, "bf16", "channel", axis=1, code="u8", symmetric=False)
    qe, se, ze = orc.quant_int(x, "bf16", "group", axis=0, group_size=6, code="u8", symmetric=False)
    assert (qd == qe).all() and (sd == se.ravel()).all() and (zd == ze.ravel()).all()
    # 1-D: PerChannel == Group{group_size: 1}
    v = workloads.normal((33,), 1.0, 22, "f32")
    q1, s1, _ = orc.quant_int(v, "f32", "channel", axis=0, code="s8")
    q2, s2, _ = orc.quant_int(v, "f32", "group", axis=0, group_size=1, code="s8")
    assert (q1 == q2).all() and (s1 == s2).all()
    # FP8 1x128 on [M,128] == one block per row; 128x128 on [128,128] == whole tensor
    y = workloads.normal((128, 128), 1.0, 23, "bf16")
    qr, sr = orc.quant_fp8_block(y, "bf16", 1, 128)
    qt, st = orc.quant_fp8_block(y, "bf16", 128, 128)
    amax_rows = np.abs(_values(y, "bf16")).max(axis=1)
    assert (sr.ravel() == (amax_rows / np.float32(448)).astype(np.float32)).all()
    assert st[0, 0] == np.float32(np.abs(_values(y, "bf16")).max() / np.float32(448))


def test_row_independence_and_permutation(orc):
    x = workloads.make_input("c2_per_token_s8", rows=64)
    q, s, _ = orc.quant_int(x, "bf16", "token", code="s8")
    q5, s5, _ = orc.quant_int(np.ascontiguousarray(x[5:9]), "bf16", "token", code="s8")
    assert (q5 == q[5:9]).all() and (s5 == s[5:9]).all()
    perm = np.random.default_rng(0).permutation(64)
    qp, sp, _ = orc.quant_int(np.ascontiguousarray(x[perm]), "bf16", "token", code="s8")
    assert (qp == q[perm]).all() and (sp == s[perm]).all()
    w = workloads.make_input("c3_per_group_u4_g128", rows=8)
    qw, sw, zw = orc.quant_int(w, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    part = np.ascontiguousarray(w[:, 256:512])
    qv, sv, zv = orc.quant_int(part, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    assert (qv == qw[:, 128:256]).all() and (sv == sw[:, 2:4]).all() and (zv == zw[:, 2:4]).all()
    for kind in ("nvfp4", "mxfp4"):
        p, b, g = orc.quant_fp4_block(x, "bf16", kind, static_global=0.01 if kind == "nvfp4" else None)
        p2, b2, _ = orc.quant_fp4_block(np.ascontiguousarray(x[7:8]), "bf16", kind,
                                        static_global=0.01 if kind == "nvfp4" else None)
        assert (p2 == p[7:8]).all() and (b2 == b[7:8]).all()


def test_requantize_is_idempotent(orc):
    x = workloads.normal((16, 256), 1.0, 31, "bf16")
    for code, sym, gran, kw in [("s8", True, "token", {}), ("u4", False, "group", dict(axis=1, group_size=128)),
                                ("u8", False, "tensor", {})]:
        q, s, z = orc.quant_int(x, "bf16", gran, code=code, symmetric=sym, **kw)
        y = orc.dequant_int(q, code, x.shape, gran, kw.get("axis", 0), kw.get("group_size", 0), s, z, "f32")
        q2, _, _ = orc.quant_int(y, "f32", gran, code=code, symmetric=sym, scale=s, zp=z, **kw)
        assert (q2 == q).all(), code


def test_transpose_for_gemm_layout(orc):
    x = workloads.normal((48, 64), 0.02, 41, "bf16")
    for kind, gs in (("nvfp4", 16), ("mxfp4", 32)):
        p, b, _ = orc.quant_fp4_block(x, "bf16", kind)
        pt, bt = orc.fp4_transpose_for_gemm(p, b, 48, 64, gs)
        assert pt.shape == (32, 48) and bt.shape == (64 // gs, 48)
        assert (pt == p.T).all() and (bt == b.T).all()


def test_degenerate_groups(orc):
    x = np.zeros((2, 128), np.float32)
    x[1, 5] = -3.0
    q, s, _ = orc.quant_int(x, "f32", "token", code="s8")
    assert s[0] == 1.0 and (q[0] == 0).all()                  # all-zero row: scale 1, codes 0
    assert _unpack(q, "s8", x.shape)[1, 5] == -127
    dy = np.full((2, 128), -2.0, np.float32)
    dx = orc.quant_int_backward(x, "f32", "token", code="s8", scale=s, dy=dy)
    assert (dx[0] == -2.0).all()                              # in range, scale 1
    qa, sa, za = orc.quant_int(x, "f32", "token", code="u8", symmetric=False)
    assert sa[0] == 1.0 and za[0] == 0 and (qa[0] == 0).all()
    y = orc.dequant_int(qa, "u8", x.shape, "token", scale=sa, zp=za, yt="f32")
    assert (y[0] == 0).all()
    # FP8 all-zero tile -> scale 1, codes +0
    q8, s8 = orc.quant_fp8_block(np.zeros((128, 128), np.float32), "f32", 128, 128)
    assert s8[0, 0] == 1.0 and (q8 == 0).all()
    # NVFP4: a block whose E4M3 scale underflows takes 0x38 (1.0)
    z = np.zeros((1, 32), np.float32)
    z[0, 0] = 1000.0
    z[0, 16] = 1e-6
    p, bs, sg = orc.quant_fp4_block(z, "f32", "nvfp4")
    assert bs[0, 1] == 0x38 and (p[0, 8:] == 0).all()
    # MXFP4 all-zero block -> E8M0 127
    p, bs, _ = orc.quant_fp4_block(np.zeros((1, 32), np.float32), "f32", "mxfp4")
    assert bs[0, 0] == 127 and (p == 0).all()
    # exact ties k + 1/2 go to the even code
    t = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]], np.float32)
    qt, st, _ = orc.quant_int(t, "f32", "token", code="s8")
    assert st[0] == 1.0
    assert list(_unpack(qt, "s8", t.shape)[0]) == [127, 0, 2, 2, 0, -2, -2, 126]


def test_zero_point_represents_zero_exactly(orc):
    x = workloads.normal((32, 256), 0.02, 51, "f16")
    q, s, z = orc.quant_int(x, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)
    # dequantizing the zero-point code gives exactly 0 and every group's
    # [min, max] lies inside the representable range (within half a step)
    xv = _values(x, "f16").reshape(32, 2, 128)
    lo = (0 - z.astype(np.float64)) * s
    hi = (15 - z.astype(np.float64)) * s
    assert (xv.min(axis=2) >= lo - s / 2).all() and (xv.max(axis=2) <= hi + s / 2).all()


@pytest.mark.parametrize("shape,block,xt", [((5, 300), (1, 128), "bf16"), ((200, 130), (128, 128), "f32"),
                                            ((7, 9), (4, 4), "f16")])
def test_bruteforce_fp8_partial_tiles(orc, shape, block, xt):
    """Shapes the blocks do not tile: the edge blocks cover only the
    elements that exist; scales are [ceil(rows/br), ceil(cols/bc)]."""
    x = workloads.normal(shape, 3.0, 78, xt)
    q, s = orc.quant_fp8_block(x, xt, *block)
    xv = _values(x, xt)
    mags = bf.e4m3_magnitudes()
    br, bc = block
    nbr, nbc = -(-shape[0] // br), -(-shape[1] // bc)
    assert s.shape == (nbr, nbc)
    for i in range(nbr):
        for j in range(nbc):
            blk = xv[i * br:min((i + 1) * br, shape[0]), j * bc:min((j + 1) * bc, shape[1])]
            sc = bf.div32(np.abs(blk).max(), 448)
            sc = np.float32(1) if sc == 0 else sc
            assert s[i, j].view(np.uint32) == sc.view(np.uint32)
            want = bf.nearest_code(bf.div32(blk, sc), mags, 0x80)
            assert (q[i * br:(i + 1) * br, j * bc:(j + 1) * bc] == want).all()
    srep = np.repeat(np.repeat(s, br, 0), bc, 1)[:shape[0], :shape[1]]
    y = orc.dequant_fp8_block(q, br, bc, s, "f32")
    dec = np.zeros(256, np.float32)
    dec[:127], dec[128:255] = mags, -mags
    assert (y == bf.mul32(dec[q], srep)).all()


@pytest.mark.parametrize("xt,static", [("bf16", None), ("f32", None), ("f16", 0.004), ("bf16", 1e-3)])
def test_fp8_per_tensor(orc, xt, static):
    """Per-tensor FP8: a dynamic scale equals the single-block FP8 result
    (one 1 x numel block); every code is the brute-force nearest E4M3 value
    of x / scale, saturating (static scales drive many codes to +-448)."""
    x = workloads.normal((12, 40), 1.0, 91, xt)
    q, s = orc.quant_fp8_per_tensor(x, xt, None if static is None else np.float32(static))
    xv = _values(x, xt)
    if static is None:
        want_s = bf.div32(np.abs(xv).max(), 448)
        assert s[0].view(np.uint32) == want_s.view(np.uint32)
        qb, sb = orc.quant_fp8_block(x.reshape(1, -1), xt, 1, x.size)
        assert (qb.reshape(q.shape) == q).all() and sb.ravel()[0] == s[0]
    else:
        assert s[0] == np.float32(static)
    want = bf.nearest_code(bf.div32(xv, s[0]), bf.e4m3_magnitudes(), 0x80)
    assert (q == want).all()
    if static is not None:
        assert ((q & 0x7F) == 0x7E).sum() > 10


# ------------------------------------------------------------ subnormal scales
def test_subnormal_symmetric_scale_clamps(orc):
    """A group whose amax lies below qmax * 2^-126 gets a subnormal scale
    with a large relative error, so |x / scale| can pass qmax: worked by
    hand, amax = 190 * 2^-149 gives scale = RN(190/127 * 2^-149) = 2^-149
    (1.496 rounds to 1 on the subnormal grid), x / scale = 190 and the code
    clamps to 127 (s8) or 7 (s4); -amax gives -127 / -7."""
    tiny = np.float32(2.0 ** -149)
    x = np.zeros((2, 16), np.float32)
    x[0, 3] = np.float32(190) * tiny
    x[1, 5] = -np.float32(190) * tiny
    x[1, 6] = np.float32(64) * tiny                 # 64 / 1 -> 64 (inside s8, clamps in s4)
    q, s, _ = orc.quant_int(x, "f32", "token", code="s8")
    assert (s.view(np.uint32) == 1).all()
    c = q.view(np.int8).reshape(2, 16)
    assert c[0, 3] == 127 and c[1, 5] == -127 and c[1, 6] == 64
    assert (np.delete(c[0], 3) == 0).all()
    q4, s4, _ = orc.quant_int(x, "f32", "token", code="s4")
    c4 = _unpack(q4, "s4", (2, 16))
    assert (s4.view(np.uint32) == np.float32(190 / 7 * 2.0 ** -149).view(np.uint32)).all()
    # 190 / 7 = 27.14 -> scale 27 * 2^-149: codes rne(190/27) = 7, rne(64/27) = 2
    assert s4[0].view(np.uint32) == 27
    assert c4[0, 3] == 7 and c4[1, 5] == -7 and c4[1, 6] == 2
