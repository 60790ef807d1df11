"""CPU oracle for scaled quantize / dequantize / STE backward.

TEST INFRASTRUCTURE ONLY.  The product path (``tensor_quantization_amd``)
never imports this package; only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It wraps ``tq_oracle.c``
(plain scalar C, binary32 arithmetic, ``-ffp-contract=off``) with numpy
arrays.  Float tensors of type f16 / bf16 are passed as ``uint16`` bit
patterns, f32 as ``float32``.

Every function states the definition it follows in ``tq_oracle.c``; the
readings taken where the pages are silent are documented there.  Functions
pinned to outside facts are listed in the tests (``tests/test_oracle_*.py``);
the choices the pages leave open (NVFP4 scale bits, MX clipping, the
asymmetric formula, degenerate groups) have no printed value to compare
with and are pinned by brute-force re-derivation on tiny tensors, closed
forms and special cases there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
# TQ_ORACLE_SANITIZE=1 builds and loads a separate copy instrumented with
# AddressSanitizer and UndefinedBehaviorSanitizer (host code only; the
# process must preload the ASan runtime, e.g.
#   TQ_ORACLE_SANITIZE=1 ASAN_OPTIONS=detect_leaks=0 \
#   LD_PRELOAD=$(gcc -print-file-name=libasan.so) python -m pytest tests -m "not gpu"
# ); any report aborts the run.
_SANITIZE = os.environ.get("TQ_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")

FTYPES = {"f32": 0, "f16": 1, "bf16": 2}
CODES = {"s8": 0, "u8": 1, "s4": 2, "u4": 3}
GRANS = {"tensor": 0, "channel": 1, "token": 2, "group": 3}
FP4_KINDS = {"nvfp4": 0, "mxfp4": 1}
FP4_GROUP = {"nvfp4": 16, "mxfp4": 32}

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, *(_SAN_FLAGS if _SANITIZE else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape_arr(shape):
    return (ctypes.c_int64 * len(shape))(*shape)


def _storage(ft):
    return np.float32 if ft == "f32" else np.uint16


def _check_float(x, ft):
    assert x.dtype == _storage(ft), (x.dtype, ft)
    return np.ascontiguousarray(x)


def code_bits(code):
    return 4 if code in ("s4", "u4") else 8


def default_q_range(code, symmetric):
    """docs.rs quantize::default_q_range (S8 [-128,127], U8 [0,255]), the
    4-bit widths alongside, and the symmetric reading [-qmax, qmax]."""
    qmin, qmax = ctypes.c_int(), ctypes.c_int()
    rc = lib().orc_default_q_range(CODES[code], int(bool(symmetric)), ctypes.byref(qmin), ctypes.byref(qmax))
    if rc:
        raise ValueError("no default range for %s symmetric=%s" % (code, symmetric))
    return qmin.value, qmax.value


def packed_shape(shape, code):
    shape = tuple(shape)
    if code_bits(code) == 4:
        return shape[:-1] + (shape[-1] // 2,)
    return shape


def scale_shape(shape, gran, axis=0, group_size=0):
    shape = tuple(shape)
    if gran == "tensor":
        return (1,)
    if gran == "token":
        return (int(np.prod(shape[:-1], dtype=np.int64)),)
    if gran == "channel":
        return (shape[axis],)
    s = list(shape)
    s[axis] //= group_size
    return tuple(s)


def _gran_args(gran, axis, group_size):
    return GRANS[gran], int(axis), int(group_size)


# ----------------------------------------------------------------- integer
def quant_int(x, xt, gran, axis=0, group_size=0, code="s8", qmin=None, qmax=None,
              symmetric=True, scale=None, zp=None):
    """Quantize to integer codes.  Returns (q, scale, zp); q is packed two
    per byte along the last dim for 4-bit codes; zp is None if symmetric.
    Pass ``scale`` (and ``zp``) to quantize with static parameters."""
    x = _check_float(x, xt)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    sshape = scale_shape(x.shape, gran, axis, group_size)
    static = scale is not None
    q = np.zeros(packed_shape(x.shape, code), np.uint8)
    s = np.ascontiguousarray(scale, np.float32).copy() if static else np.zeros(sshape, np.float32)
    if symmetric:
        z = None
    else:
        z = np.ascontiguousarray(zp).view(np.uint8).copy() if static else np.zeros(sshape, np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_quant_int(_p(x), FTYPES[xt], x.ndim, _shape_arr(x.shape), g, a,
                             ctypes.c_int64(gsz), CODES[code], qmin, qmax, int(bool(symmetric)),
                             int(static), _p(q), _p(s), _p(z))
    if rc:
        raise ValueError("oracle rejected quant_int arguments")
    if z is not None and code in ("s8", "s4"):
        z = z.view(np.int8)
    return q, s, z


def dequant_int(q, code, shape, gran, axis=0, group_size=0, scale=None, zp=None, yt="f32"):
    q = np.ascontiguousarray(q, np.uint8)
    y = np.zeros(tuple(shape), _storage(yt))
    zpa = None if zp is None else np.ascontiguousarray(zp).view(np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_dequant_int(_p(q), CODES[code], len(shape), _shape_arr(shape), g, a,
                               ctypes.c_int64(gsz), _p(np.ascontiguousarray(scale, np.float32)),
                               _p(zpa), _p(y), FTYPES[yt])
    if rc:
        raise ValueError("oracle rejected dequant_int arguments")
    return y


def quant_int_backward(x, xt, gran, axis=0, group_size=0, code="s8", qmin=None, qmax=None,
                       symmetric=True, scale=None, zp=None, dy=None):
    x = _check_float(x, xt)
    dy = _check_float(dy, xt)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    dx = np.zeros(x.shape, _storage(xt))
    zpa = None if zp is None else np.ascontiguousarray(zp).view(np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_quant_int_backward(_p(x), FTYPES[xt], x.ndim, _shape_arr(x.shape), g, a,
                                      ctypes.c_int64(gsz), qmin, qmax,
                                      _p(np.ascontiguousarray(scale, np.float32)), _p(zpa),
                                      CODES[code], _p(dy), _p(dx))
    if rc:
        raise ValueError("oracle rejected quant_int_backward arguments")
    return dx


def dequant_int_backward(dy, dyt, gran, axis=0, group_size=0, scale=None):
    dy = _check_float(dy, dyt)
    dq = np.zeros(dy.shape, _storage(dyt))
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_dequant_int_backward(_p(dy), FTYPES[dyt], dy.ndim, _shape_arr(dy.shape), g, a,
                                        ctypes.c_int64(gsz),
                                        _p(np.ascontiguousarray(scale, np.float32)), _p(dq))
    if rc:
        raise ValueError("oracle rejected dequant_int_backward arguments")
    return dq


# ----------------------------------------------------------------- FP8
def quant_fp8_block(x, xt, block_rows, block_cols):
    x = _check_float(x, xt)
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.uint8)
    s = np.zeros((-(-rows // block_rows), -(-cols // block_cols)), np.float32)
    rc = lib().orc_quant_fp8_block(_p(x), FTYPES[xt], ctypes.c_int64(rows), ctypes.c_int64(cols),
                                   ctypes.c_int64(block_rows), ctypes.c_int64(block_cols), _p(q), _p(s))
    if rc:
        raise ValueError("oracle rejected quant_fp8_block arguments")
    return q, s


def dequant_fp8_block(q, block_rows, block_cols, scale, yt):
    q = np.ascontiguousarray(q, np.uint8)
    rows, cols = q.shape
    y = np.zeros((rows, cols), _storage(yt))
    rc = lib().orc_dequant_fp8_block(_p(q), ctypes.c_int64(rows), ctypes.c_int64(cols),
                                     ctypes.c_int64(block_rows), ctypes.c_int64(block_cols),
                                     _p(np.ascontiguousarray(scale, np.float32)), _p(y), FTYPES[yt])
    if rc:
        raise ValueError("oracle rejected dequant_fp8_block arguments")
    return y


def quant_fp8_block_backward(x, xt, block_rows, block_cols, scale, dy):
    x = _check_float(x, xt)
    dy = _check_float(dy, xt)
    rows, cols = x.shape
    dx = np.zeros((rows, cols), _storage(xt))
    rc = lib().orc_quant_fp8_block_backward(_p(x), FTYPES[xt], ctypes.c_int64(rows), ctypes.c_int64(cols),
                                            ctypes.c_int64(block_rows), ctypes.c_int64(block_cols),
                                            _p(np.ascontiguousarray(scale, np.float32)), _p(dy), _p(dx))
    if rc:
        raise ValueError("oracle rejected quant_fp8_block_backward arguments")
    return dx


def dequant_fp8_block_backward(dy, dyt, block_rows, block_cols, scale):
    dy = _check_float(dy, dyt)
    rows, cols = dy.shape
    dq = np.zeros((rows, cols), _storage(dyt))
    rc = lib().orc_dequant_fp8_block_backward(_p(dy), FTYPES[dyt], ctypes.c_int64(rows), ctypes.c_int64(cols),
                                              ctypes.c_int64(block_rows), ctypes.c_int64(block_cols),
                                              _p(np.ascontiguousarray(scale, np.float32)), _p(dq))
    if rc:
        raise ValueError("oracle rejected dequant_fp8_block_backward arguments")
    return dq


# ----------------------------------------------------------------- FP4
def quant_fp4_block(x, xt, kind, static_global=None):
    """Returns (packed [rows, K/2] u8, block scales [rows, K/gs] u8,
    global scale float32 (NVFP4; 1.0 for MXFP4))."""
    x = _check_float(x, xt)
    rows, k = x.shape
    gs = FP4_GROUP[kind]
    packed = np.zeros((rows, k // 2), np.uint8)
    bs = np.zeros((rows, k // gs), np.uint8)
    sg = np.array([1.0 if static_global is None else static_global], np.float32)
    rc = lib().orc_quant_fp4_block(_p(x), FTYPES[xt], ctypes.c_int64(rows), ctypes.c_int64(k),
                                   FP4_KINDS[kind], _p(packed), _p(bs), _p(sg),
                                   int(static_global is not None))
    if rc:
        raise ValueError("oracle rejected quant_fp4_block arguments")
    return packed, bs, sg


def dequant_fp4_block(packed, bscale, global_scale, kind, yt):
    packed = np.ascontiguousarray(packed, np.uint8)
    rows, kb = packed.shape
    k = kb * 2
    y = np.zeros((rows, k), _storage(yt))
    sg = np.asarray([global_scale], np.float32).reshape(1)
    rc = lib().orc_dequant_fp4_block(_p(packed), _p(np.ascontiguousarray(bscale, np.uint8)), _p(sg),
                                     ctypes.c_int64(rows), ctypes.c_int64(k), FP4_KINDS[kind], _p(y),
                                     FTYPES[yt])
    if rc:
        raise ValueError("oracle rejected dequant_fp4_block arguments")
    return y


def quant_fp4_block_backward(x, xt, bscale, global_scale, kind, dy):
    x = _check_float(x, xt)
    dy = _check_float(dy, xt)
    rows, k = x.shape
    dx = np.zeros((rows, k), _storage(xt))
    sg = np.asarray([global_scale], np.float32).reshape(1)
    rc = lib().orc_quant_fp4_block_backward(_p(x), FTYPES[xt], _p(np.ascontiguousarray(bscale, np.uint8)),
                                            _p(sg), ctypes.c_int64(rows), ctypes.c_int64(k),
                                            FP4_KINDS[kind], _p(dy), _p(dx))
    if rc:
        raise ValueError("oracle rejected quant_fp4_block_backward arguments")
    return dx


def dequant_fp4_block_backward(dy, dyt, bscale, global_scale, kind):
    dy = _check_float(dy, dyt)
    rows, k = dy.shape
    dq = np.zeros((rows, k), _storage(dyt))
    sg = np.asarray([global_scale], np.float32).reshape(1)
    rc = lib().orc_dequant_fp4_block_backward(_p(dy), FTYPES[dyt], _p(np.ascontiguousarray(bscale, np.uint8)),
                                              _p(sg), ctypes.c_int64(rows), ctypes.c_int64(k),
                                              FP4_KINDS[kind], _p(dq))
    if rc:
        raise ValueError("oracle rejected dequant_fp4_block_backward arguments")
    return dq


def fp4_transpose_for_gemm(packed, bscale, n, k, gs):
    packed = np.ascontiguousarray(packed, np.uint8)
    bscale = np.ascontiguousarray(bscale, np.uint8)
    pt = np.zeros((k // 2, n), np.uint8)
    st = np.zeros((k // gs, n), np.uint8)
    rc = lib().orc_fp4_transpose_for_gemm(_p(packed), _p(bscale), ctypes.c_int64(n), ctypes.c_int64(k),
                                          ctypes.c_int64(gs), _p(pt), _p(st))
    if rc:
        raise ValueError("oracle rejected fp4_transpose_for_gemm arguments")
    return pt, st


# ----------------------------------------------------------------- scalars
def _map_f32(fn, v, out_dtype):
    v = np.ascontiguousarray(v, np.float32)
    out = np.zeros(v.shape, out_dtype)
    getattr(lib(), fn)(_p(v), ctypes.c_int64(v.size), _p(out))
    return out


def enc_e4m3(v):
    return _map_f32("orc_enc_e4m3_array", v, np.uint8)


def enc_e2m1(v):
    return _map_f32("orc_enc_e2m1_array", v, np.uint8)


def enc_e8m0_mx(amax):
    return _map_f32("orc_enc_e8m0_mx_array", amax, np.uint8)


def narrow_bf16(v):
    return _map_f32("orc_narrow_bf16_array", v, np.uint16)


def narrow_f16(v):
    return _map_f32("orc_narrow_f16_array", v, np.uint16)


def f16_to_f32(h):
    h = np.ascontiguousarray(h, np.uint16)
    out = np.zeros(h.shape, np.float32)
    lib().orc_f16_to_f32_array(_p(h), ctypes.c_int64(h.size), _p(out))
    return out


def bf16_to_f32(h):
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def dec_e4m3_table():
    f = lib().orc_dec_e4m3
    f.restype = ctypes.c_float
    return np.array([f(ctypes.c_uint8(c)) for c in range(256)], np.float32)


def dec_e2m1_table():
    f = lib().orc_dec_e2m1
    f.restype = ctypes.c_float
    return np.array([f(ctypes.c_uint8(c)) for c in range(16)], np.float32)


def dec_e8m0(b):
    f = lib().orc_dec_e8m0
    f.restype = ctypes.c_float
    return np.float32(f(ctypes.c_uint8(int(b))))


def widen(x, xt):
    """Float tensor storage -> float32 values (exact)."""
    if xt == "f32":
        return np.asarray(x, np.float32)
    if xt == "bf16":
        return bf16_to_f32(x)
    return f16_to_f32(x)


# ----------------------------------------------------------------- FP4 layout follow-ons
def fp4_transpose_concat(parts, k, gs, align=1):
    """parts: list of (packed [n_i, k/2], block scales [n_i, k/gs]).
    Returns (packed_t [k/2, stride], scales_t [k/gs, stride], stride)."""
    n = [int(p.shape[0]) for p, _ in parts]
    total = sum(n)
    stride = -(-total // align) * align if align > 1 else total
    pt = np.zeros((k // 2, stride), np.uint8)
    st = np.zeros((k // gs, stride), np.uint8)
    keep = [(np.ascontiguousarray(p, np.uint8), np.ascontiguousarray(b, np.uint8)) for p, b in parts]
    pp = (ctypes.c_void_p * len(keep))(*[_p(p).value for p, _ in keep])
    bb = (ctypes.c_void_p * len(keep))(*[_p(b).value for _, b in keep])
    nn = (ctypes.c_int64 * len(n))(*n)
    rc = lib().orc_fp4_transpose_concat(len(keep), pp, bb, nn, ctypes.c_int64(k), ctypes.c_int64(gs),
                                        ctypes.c_int64(stride), _p(pt), _p(st))
    if rc:
        raise ValueError("oracle rejected fp4_transpose_concat arguments")
    return pt, st, stride


def fp4_concat_rows(p1, s1, g1, p2, s2, g2, k):
    p1 = np.ascontiguousarray(p1, np.uint8)
    p2 = np.ascontiguousarray(p2, np.uint8)
    n1, n2 = p1.shape[0], p2.shape[0]
    po = np.zeros((n1 + n2, k // 2), np.uint8)
    so = np.zeros((n1 + n2, k // 16), np.uint8)
    rc = lib().orc_fp4_concat_rows(_p(p1), _p(np.ascontiguousarray(s1, np.uint8)), ctypes.c_float(g1), _p(p2),
                                   _p(np.ascontiguousarray(s2, np.uint8)), ctypes.c_float(g2),
                                   ctypes.c_int64(n1), ctypes.c_int64(n2), ctypes.c_int64(k), _p(po), _p(so))
    if rc:
        raise ValueError("oracle rejected fp4_concat_rows arguments")
    return po, so


def fp4_predequant_to_fp8(packed, bscale, global_scale, kind):
    packed = np.ascontiguousarray(packed, np.uint8)
    rows, kb = packed.shape
    out = np.zeros((rows, kb * 2), np.uint8)
    rc = lib().orc_fp4_predequant_to_fp8(_p(packed), _p(np.ascontiguousarray(bscale, np.uint8)),
                                         ctypes.c_float(global_scale), ctypes.c_int64(rows), ctypes.c_int64(kb * 2),
                                         FP4_KINDS[kind], _p(out))
    if rc:
        raise ValueError("oracle rejected fp4_predequant_to_fp8 arguments")
    return out


# ----------------------------------------------------------------- fake quantization / dynamic range
def fake_quant_per_tensor(x, xt, code="s8", qmin=None, qmax=None, symmetric=True, scale=None, zp=None):
    """Per-tensor round trip y = (q - zp) * scale in x's type.  Returns
    (y, scale float32[1], zp int8/uint8[1] or None); pass ``scale`` (and
    ``zp``) for static parameters."""
    x = _check_float(x, xt)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    static = scale is not None
    s = np.ascontiguousarray(scale, np.float32).reshape(1).copy() if static else np.zeros(1, np.float32)
    z = None
    if not symmetric:
        z = np.ascontiguousarray(zp).view(np.uint8).reshape(1).copy() if static else np.zeros(1, np.uint8)
    y = np.zeros(x.shape, _storage(xt))
    rc = lib().orc_fake_quant_per_tensor(_p(x), FTYPES[xt], ctypes.c_int64(x.size), CODES[code], qmin, qmax,
                                         int(bool(symmetric)), int(static), _p(s), _p(z), _p(y))
    if rc:
        raise ValueError("oracle rejected fake_quant_per_tensor arguments")
    if z is not None and code in ("s8", "s4"):
        z = z.view(np.int8)
    return y, s, z


def fake_quant_per_tensor_backward(x, xt, dy, scale, zp=None, code="s8", qmin=None, qmax=None, symmetric=True):
    x = _check_float(x, xt)
    dy = _check_float(dy, xt)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    dx = np.zeros(x.shape, _storage(xt))
    zpa = None if zp is None else np.ascontiguousarray(zp).view(np.uint8)
    rc = lib().orc_fake_quant_per_tensor_backward(_p(x), FTYPES[xt], ctypes.c_int64(x.size), CODES[code], qmin,
                                                  qmax, _p(np.ascontiguousarray(scale, np.float32)), _p(zpa),
                                                  _p(dy), _p(dx))
    if rc:
        raise ValueError("oracle rejected fake_quant_per_tensor_backward arguments")
    return dx


RANGE_MODES = {"symmetric": 0, "asymmetric": 1}
RANGE_SCOPES = {"tensor": 0, "token": 1, "channel": 2}


def dynamic_range_quantize(x, xt, mode, scope, code, axis=0):
    """Returns (q, scale, zp or None) with the code's default range for the
    mode and the scale tensor of the scope."""
    x = _check_float(x, xt)
    gran = {"tensor": "tensor", "token": "token", "channel": "channel"}[scope]
    sshape = scale_shape(x.shape, gran, axis)
    q = np.zeros(packed_shape(x.shape, code), np.uint8)
    s = np.zeros(sshape, np.float32)
    z = None if mode == "symmetric" else np.zeros(sshape, np.uint8)
    rc = lib().orc_dynamic_range_quantize(_p(x), FTYPES[xt], x.ndim, _shape_arr(x.shape), RANGE_MODES[mode],
                                          RANGE_SCOPES[scope], int(axis), CODES[code], _p(q), _p(s), _p(z))
    if rc:
        raise ValueError("oracle rejected dynamic_range_quantize arguments")
    if z is not None and code in ("s8", "s4"):
        z = z.view(np.int8)
    return q, s, z


# ----------------------------------------------------------------- MXFP8
def enc_e8m0_mx8(v):
    """Shared MX scale byte for E4M3 elements: floor(log2 amax) - 8 + 127."""
    return _map_f32("orc_enc_e8m0_mx8_array", v, np.uint8)


def quant_mxfp8(x, xt):
    """Returns (q [rows, k] E4M3 bytes, block scales [rows, k/32] E8M0 bytes)."""
    x = _check_float(x, xt)
    rows, k = x.shape
    q = np.zeros((rows, k), np.uint8)
    s = np.zeros((rows, k // 32), np.uint8)
    if lib().orc_quant_mxfp8(_p(x), FTYPES[xt], ctypes.c_int64(rows), ctypes.c_int64(k), _p(q), _p(s)):
        raise ValueError("oracle rejected quant_mxfp8 arguments")
    return q, s


def dequant_mxfp8(q, bscale, yt="f32"):
    q = np.ascontiguousarray(q, np.uint8)
    rows, k = q.shape
    y = np.zeros((rows, k), _storage(yt))
    if lib().orc_dequant_mxfp8(_p(q), _p(np.ascontiguousarray(bscale, np.uint8)), ctypes.c_int64(rows),
                               ctypes.c_int64(k), _p(y), FTYPES[yt]):
        raise ValueError("oracle rejected dequant_mxfp8 arguments")
    return y


def quant_mxfp8_backward(x, xt, bscale, dy):
    x = _check_float(x, xt)
    dy = _check_float(dy, xt)
    rows, k = x.shape
    dx = np.zeros(x.shape, _storage(xt))
    if lib().orc_quant_mxfp8_backward(_p(x), FTYPES[xt], _p(np.ascontiguousarray(bscale, np.uint8)),
                                      ctypes.c_int64(rows), ctypes.c_int64(k), _p(dy), _p(dx)):
        raise ValueError("oracle rejected quant_mxfp8_backward arguments")
    return dx


def dequant_mxfp8_backward(dy, dyt, bscale):
    dy = _check_float(dy, dyt)
    rows, k = dy.shape
    dq = np.zeros(dy.shape, _storage(dyt))
    if lib().orc_dequant_mxfp8_backward(_p(dy), FTYPES[dyt], _p(np.ascontiguousarray(bscale, np.uint8)),
                                        ctypes.c_int64(rows), ctypes.c_int64(k), _p(dq)):
        raise ValueError("oracle rejected dequant_mxfp8_backward arguments")
    return dq


def quant_fp8_per_tensor(x, xt, scale=None):
    """Returns (q E4M3 bytes of x's shape, scale float32[1]); ``scale`` makes
    the scale a static input."""
    x = _check_float(x, xt)
    static = scale is not None
    s = np.ascontiguousarray(scale, np.float32).reshape(1).copy() if static else np.zeros(1, np.float32)
    q = np.zeros(x.shape, np.uint8)
    if lib().orc_quant_fp8_per_tensor(_p(x), FTYPES[xt], ctypes.c_int64(x.size), int(static), _p(s), _p(q)):
        raise ValueError("oracle rejected quant_fp8_per_tensor arguments")
    return q, s


# ----------------------------------------------------------------- binary64 inputs
def quant_f64(x, gran, axis=0, group_size=0, code="s8", qmin=None, qmax=None, symmetric=True, scale=None, zp=None):
    """Binary64 quantize: x float64; returns (q, scale float64, zp or None)."""
    x = np.ascontiguousarray(x, np.float64)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    sshape = scale_shape(x.shape, gran, axis, group_size)
    static = scale is not None
    q = np.zeros(packed_shape(x.shape, code), np.uint8)
    s = np.ascontiguousarray(scale, np.float64).copy() if static else np.zeros(sshape, np.float64)
    z = None
    if not symmetric:
        z = np.ascontiguousarray(zp).view(np.uint8).copy() if static else np.zeros(sshape, np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_quant_f64(_p(x), x.ndim, _shape_arr(x.shape), g, a, ctypes.c_int64(gsz), CODES[code], qmin, qmax,
                             int(bool(symmetric)), int(static), _p(q), _p(s), _p(z))
    if rc:
        raise ValueError("oracle rejected quant_f64 arguments")
    if z is not None and code in ("s8", "s4"):
        z = z.view(np.int8)
    return q, s, z


def dequant_f64(q, code, shape, gran, axis=0, group_size=0, scale=None, zp=None):
    q = np.ascontiguousarray(q, np.uint8)
    y = np.zeros(tuple(shape), np.float64)
    zpa = None if zp is None else np.ascontiguousarray(zp).view(np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_dequant_f64(_p(q), CODES[code], len(shape), _shape_arr(shape), g, a, ctypes.c_int64(gsz),
                               _p(np.ascontiguousarray(scale, np.float64)), _p(zpa), _p(y))
    if rc:
        raise ValueError("oracle rejected dequant_f64 arguments")
    return y


def quant_f64_backward(x, gran, axis=0, group_size=0, code="s8", qmin=None, qmax=None, symmetric=True, scale=None,
                       zp=None, dy=None):
    x = np.ascontiguousarray(x, np.float64)
    dy = np.ascontiguousarray(dy, np.float64)
    if qmin is None:
        qmin, qmax = default_q_range(code, symmetric)
    dx = np.zeros(x.shape, np.float64)
    zpa = None if zp is None else np.ascontiguousarray(zp).view(np.uint8)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_quant_f64_backward(_p(x), x.ndim, _shape_arr(x.shape), g, a, ctypes.c_int64(gsz), CODES[code],
                                      qmin, qmax, _p(np.ascontiguousarray(scale, np.float64)), _p(zpa), _p(dy),
                                      _p(dx))
    if rc:
        raise ValueError("oracle rejected quant_f64_backward arguments")
    return dx


def dequant_f64_backward(dy, gran, axis=0, group_size=0, scale=None):
    dy = np.ascontiguousarray(dy, np.float64)
    dq = np.zeros(dy.shape, np.float64)
    g, a, gsz = _gran_args(gran, axis, group_size)
    rc = lib().orc_dequant_f64_backward(_p(dy), dy.ndim, _shape_arr(dy.shape), g, a, ctypes.c_int64(gsz),
                                        _p(np.ascontiguousarray(scale, np.float64)), _p(dq))
    if rc:
        raise ValueError("oracle rejected dequant_f64_backward arguments")
    return dq


# ----------------------------------------------------------------- FP8 block GEMM
def fp8_block_gemm(qa, sa, qw, sw):
    """qa [M, K] E4M3, sa [M, K/128] f32, qw [N, K] E4M3, sw [N/128, K/128] f32.
    Returns (y [M, N] float64, yabs [M, N] float64)."""
    qa = np.ascontiguousarray(qa, np.uint8)
    qw = np.ascontiguousarray(qw, np.uint8)
    M, K = qa.shape
    N = qw.shape[0]
    y = np.zeros((M, N), np.float64)
    ya = np.zeros((M, N), np.float64)
    rc = lib().orc_fp8_block_gemm(_p(qa), _p(np.ascontiguousarray(sa, np.float32)), _p(qw),
                                  _p(np.ascontiguousarray(sw, np.float32)), ctypes.c_int64(M), ctypes.c_int64(N),
                                  ctypes.c_int64(K), _p(y), _p(ya))
    if rc:
        raise ValueError("oracle rejected fp8_block_gemm arguments")
    return y, ya


def w8a8_linear(qx, sx, qw, sw, yt):
    """qx [M, K] s8, sx [M] f32, qw [N, K] s8, sw [N] f32 -> y [M, N] in yt
    (f32 values, or bf16 / f16 bit patterns as uint16)."""
    qx = np.ascontiguousarray(qx, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, K = qx.shape
    N = qw.shape[0]
    y = np.zeros((M, N), np.float32 if yt == "f32" else np.uint16)
    rc = lib().orc_w8a8_linear(_p(qx), _p(np.ascontiguousarray(sx, np.float32)), _p(qw),
                               _p(np.ascontiguousarray(sw, np.float32)), ctypes.c_int64(M), ctypes.c_int64(N),
                               ctypes.c_int64(K), _p(y), FTYPES[yt])
    if rc:
        raise ValueError("oracle rejected w8a8_linear arguments")
    return y


def fp4_linear(x, packed, bscale, global_scale, kind):
    """x bf16 bits [M, K] (uint16), packed [N, K/2], bscale [N, K/gs] (E4M3
    bytes for NVFP4, E8M0 for MXFP4), global_scale (NVFP4).  Returns
    (y [M, N] float64, yabs [M, N] float64)."""
    x = np.ascontiguousarray(x, np.uint16)
    packed = np.ascontiguousarray(packed, np.uint8)
    M, K = x.shape
    N = packed.shape[0]
    y = np.zeros((M, N), np.float64)
    ya = np.zeros((M, N), np.float64)
    rc = lib().orc_fp4_linear(_p(x), _p(packed), _p(np.ascontiguousarray(bscale, np.uint8)),
                              ctypes.c_float(float(np.asarray(global_scale).reshape(-1)[0])), FP4_KINDS[kind], ctypes.c_int64(M),
                              ctypes.c_int64(N), ctypes.c_int64(K), _p(y), _p(ya))
    if rc:
        raise ValueError("oracle rejected fp4_linear arguments")
    return y, ya
