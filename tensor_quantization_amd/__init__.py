"""Python binding of the gfx950 quantization library (``libtq.so``).

Argument marshalling only: every function here has the name of the C entry
point it calls (``include/tq.h``), allocates the output tensors with torch on
the input's device, passes raw device pointers and the current HIP stream,
and raises ``TQError`` on a non-zero status.  All arithmetic runs in the HIP
kernels; there is no CPU fallback: importing this package without the built
library raises.

Float tensors are torch.float32 / float16 / bfloat16.  Integer codes are
named 's8', 'u8', 's4', 'u4'; 4-bit codes come back packed two per byte along
the last dimension (even index in the low nibble).  Zero-points are int8 for
signed codes and uint8 for unsigned ones; ``None`` means symmetric.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "tensor_quantization_amd: %s is missing; build it with "
        "`python tensor_quantization_amd/build.py` (hipcc, gfx950)" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_ALIGN, TQ_ERR_HIP = range(5)
FTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
CODE = {"s8": 0, "u8": 1, "s4": 2, "u4": 3}
FP4_KIND = {"nvfp4": 0, "mxfp4": 1}
FP4_GROUP = {"nvfp4": 16, "mxfp4": 32}

_P = ctypes.c_void_p
_I = ctypes.c_int
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SHAPE = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "tq_abi_version": ([], _I),
    "tq_status_str": ([_I], ctypes.c_char_p),
    "tq_default_q_range": ([_I, _I, ctypes.POINTER(_I32), ctypes.POINTER(_I32)], _I),
    "tq_workspace_bytes": ([_I, _I64], _SZ),
    "tq_quant_per_tensor": ([_P, _I, _I64, _I, _I32, _I32, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "tq_quant_per_channel": ([_P, _I, _I32, _SHAPE, _I32, _I, _I32, _I32, _P, _P, _P, _P], _I),
    "tq_quant_per_token": ([_P, _I, _I64, _I64, _I, _I32, _I32, _P, _P, _P, _P], _I),
    "tq_quant_per_group": ([_P, _I, _I32, _SHAPE, _I32, _I64, _I, _I32, _I32, _P, _P, _P, _P], _I),
    "tq_dequant_per_tensor": ([_P, _I, _I64, _P, _P, _P, _I, _P], _I),
    "tq_dequant_per_channel": ([_P, _I, _I32, _SHAPE, _I32, _P, _P, _P, _I, _P], _I),
    "tq_dequant_per_token": ([_P, _I, _I64, _I64, _P, _P, _P, _I, _P], _I),
    "tq_dequant_per_group": ([_P, _I, _I32, _SHAPE, _I32, _I64, _P, _P, _P, _I, _P], _I),
    "tq_quant_per_tensor_backward": ([_P, _I, _I64, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_quant_per_channel_backward": ([_P, _I, _I32, _SHAPE, _I32, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_quant_per_token_backward": ([_P, _I, _I64, _I64, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_quant_per_group_backward": ([_P, _I, _I32, _SHAPE, _I32, _I64, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_dequant_per_tensor_backward": ([_P, _I, _I64, _P, _P, _P], _I),
    "tq_dequant_per_channel_backward": ([_P, _I, _I32, _SHAPE, _I32, _P, _P, _P], _I),
    "tq_dequant_per_token_backward": ([_P, _I, _I64, _I64, _P, _P, _P], _I),
    "tq_dequant_per_group_backward": ([_P, _I, _I32, _SHAPE, _I32, _I64, _P, _P, _P], _I),
    "tq_quant_fp8_block": ([_P, _I, _I64, _I64, _I32, _I32, _P, _P, _P], _I),
    "tq_dequant_fp8_block": ([_P, _I64, _I64, _I32, _I32, _P, _P, _I, _P], _I),
    "tq_quant_fp8_block_backward": ([_P, _I, _I64, _I64, _I32, _I32, _P, _P, _P, _P], _I),
    "tq_dequant_fp8_block_backward": ([_P, _I, _I64, _I64, _I32, _I32, _P, _P, _P], _I),
    "tq_quant_fp4_block": ([_P, _I, _I64, _I64, _I, _P, _P, _P, _I, _P, _SZ, _P], _I),
    "tq_quant_fp4_block_noalloc": ([_P, _I, _I64, _I64, _I, _P, _P, _P, _I, _P], _I),
    "tq_dequant_fp4_block": ([_P, _P, _P, _I64, _I64, _I, _P, _I, _P], _I),
    "tq_quant_fp4_block_backward": ([_P, _I, _P, _P, _I64, _I64, _I, _P, _P, _P], _I),
    "tq_dequant_fp4_block_backward": ([_P, _I, _P, _P, _I64, _I64, _I, _P, _P], _I),
    "tq_fp4_transpose_for_gemm": ([_P, _P, _I64, _I64, _I32, _P, _P, _P], _I),
    "tq_fp4_transpose_concat_for_gemm": ([_I32, ctypes.POINTER(_P), ctypes.POINTER(_P), _SHAPE, _I64, _I32, _I64,
                                          _P, _P, ctypes.POINTER(_I64), _P], _I),
    "tq_fp4_concat_rows": ([_P, _P, ctypes.c_float, _P, _P, ctypes.c_float, _I64, _I64, _I64, _P, _P, _P], _I),
    "tq_fp4_predequant_to_fp8": ([_P, _P, ctypes.c_float, _I64, _I64, _I, _P, _P], _I),
    "tq_fake_quant_per_tensor": ([_P, _I, _I64, _I, _I32, _I32, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "tq_fake_quant_per_tensor_backward": ([_P, _I, _I64, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_dynamic_range_quantize": ([_P, _I, _I32, _SHAPE, _I, _I, _I32, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "tq_quant_mxfp8": ([_P, _I, _I64, _I64, _P, _P, _P], _I),
    "tq_quant_fp8_per_tensor": ([_P, _I, _I64, _I, _P, _P, _P, _SZ, _P], _I),
    "tq_dequant_fp8_per_tensor": ([_P, _I64, _P, _P, _I, _P], _I),
    "tq_quant_per_token_strided": ([_P, _I, _I64, _I64, _I64, _I, _I32, _I32, _P, _P, _P, _P], _I),
    "tq_quant_fp8_rows_strided": ([_P, _I, _I64, _I64, _I64, _I32, _P, _P, _P], _I),
    "tq_fp8_block_gemm": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "tq_w8a8_linear": ([_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P], _I),
    "tq_fp4_linear": ([_P, _I, _P, _P, _P, _I, _I64, _I64, _I64, _P, _I, _P], _I),
    "tq_quant_f64": ([_P, _I32, _SHAPE, _I, _I32, _I64, _I, _I32, _I32, _I, _P, _P, _P, _P, _SZ, _P], _I),
    "tq_dequant_f64": ([_P, _I, _I32, _SHAPE, _I, _I32, _I64, _P, _P, _P, _P], _I),
    "tq_quant_f64_backward": ([_P, _I32, _SHAPE, _I, _I32, _I64, _I, _I32, _I32, _P, _P, _P, _P, _P], _I),
    "tq_dequant_f64_backward": ([_P, _I32, _SHAPE, _I, _I32, _I64, _P, _P, _P], _I),
    "tq_dequant_mxfp8": ([_P, _P, _I64, _I64, _P, _I, _P], _I),
    "tq_quant_mxfp8_backward": ([_P, _I, _P, _I64, _I64, _P, _P, _P], _I),
    "tq_dequant_mxfp8_backward": ([_P, _I, _P, _I64, _I64, _P, _P], _I),
    "tq_stream_mix": ([_P, _P, _I64, _I, _I, _I, _I, _P], _I),
}

for _name, (_args, _ret) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _ret

EXPORTED = tuple(_SIGS)


class TQError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s: %s (status %d)" % (fn, _lib.tq_status_str(status).decode(), status))
        self.status = status


def _call(name, *args):
    rc = getattr(_lib, name)(*args)
    if rc != TQ_OK:
        raise TQError(name, rc)


# ------------------------------------------------------------ marshalling
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ft(t):
    try:
        return FTYPE[t.dtype]
    except KeyError:
        raise TypeError("unsupported float dtype %s" % t.dtype) from None


def _dev_float(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    _ft(t)
    return t.contiguous()


def _shape(shape):
    arr = (ctypes.c_int64 * len(shape))(*[int(s) for s in shape])
    return arr, len(shape)


def _bits(code):
    return 4 if code in ("s4", "u4") else 8


def _zp_dtype(code):
    return torch.int8 if code in ("s8", "s4") else torch.uint8


def _packed_shape(shape, code):
    shape = tuple(shape)
    if _bits(code) == 4:
        if not shape or shape[-1] % 2:
            raise ValueError("4-bit codes need an even last dimension")
        return shape[:-1] + (shape[-1] // 2,)
    return shape


def tq_abi_version():
    return _lib.tq_abi_version()


def tq_default_q_range(code, symmetric):
    lo, hi = _I32(), _I32()
    _call("tq_default_q_range", CODE[code], int(bool(symmetric)), ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def tq_workspace_bytes(op, numel):
    return int(_lib.tq_workspace_bytes(op, numel))


def tq_stream_mix(src, dst, nthreads, in_bytes, out_bytes, policy=1, vectors=1):
    """Measurement utility: the streaming ceiling of an access mix (each of
    `nthreads` units reads `in_bytes` of src and writes `out_bytes` of dst;
    a lane takes `vectors` units)."""
    _call("tq_stream_mix", _ptr(src), _ptr(dst), int(nthreads), int(in_bytes), int(out_bytes), int(policy),
          int(vectors), _stream(src.device))


def _range(code, qmin, qmax, symmetric):
    if qmin is None or qmax is None:
        lo, hi = tq_default_q_range(code, symmetric)
        qmin = lo if qmin is None else qmin
        qmax = hi if qmax is None else qmax
    return int(qmin), int(qmax)


def _scale_shape(shape, axis, group_size):
    s = list(shape)
    s[axis] //= group_size
    return tuple(s)


def _outputs(x, code, sshape, symmetric):
    dev = x.device
    q = torch.empty(_packed_shape(x.shape, code), dtype=torch.uint8, device=dev)
    scale = torch.empty(sshape, dtype=torch.float32, device=dev)
    zp = None if symmetric else torch.empty(sshape, dtype=_zp_dtype(code), device=dev)
    return q, scale, zp


# ------------------------------------------------------------ integer quantize
def tq_quant_per_tensor(x, code="s8", qmin=None, qmax=None, symmetric=True, scale=None, zero_point=None):
    """Per-tensor quantize.  Passing ``scale`` (and ``zero_point``) makes
    them static inputs; otherwise they are computed and returned."""
    x = _dev_float(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    static = scale is not None
    q, s, z = _outputs(x, code, (1,), symmetric)
    if static:
        s = scale.to(device=x.device, dtype=torch.float32).reshape(1).contiguous()
        if not symmetric:
            z = zero_point.to(device=x.device, dtype=_zp_dtype(code)).reshape(1).contiguous()
    ws = torch.empty(max(1, tq_workspace_bytes(0, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_quant_per_tensor", _ptr(x), _ft(x), x.numel(), CODE[code], qmin, qmax, int(static), _ptr(q),
          _ptr(s), _ptr(z), _ptr(ws), ws.numel(), _stream(x.device))
    return q, s, z


def tq_quant_per_channel(x, axis=0, code="s8", qmin=None, qmax=None, symmetric=True):
    x = _dev_float(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    q, s, z = _outputs(x, code, (x.shape[axis],), symmetric)
    shp, nd = _shape(x.shape)
    _call("tq_quant_per_channel", _ptr(x), _ft(x), nd, shp, axis, CODE[code], qmin, qmax, _ptr(q), _ptr(s),
          _ptr(z), _stream(x.device))
    return q, s, z


def tq_quant_per_token(x, code="s8", qmin=None, qmax=None, symmetric=True):
    """Per-token (per-row) quantize of x viewed as [rows, cols] (leading
    dimensions flattened); scale has one entry per row."""
    x = _dev_float(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    q, s, z = _outputs(x, code, (rows,), symmetric)
    _call("tq_quant_per_token", _ptr(x), _ft(x), rows, cols, CODE[code], qmin, qmax, _ptr(q), _ptr(s),
          _ptr(z), _stream(x.device))
    return q, s, z


def tq_quant_per_group(x, axis=-1, group_size=128, code="u4", qmin=None, qmax=None, symmetric=False):
    x = _dev_float(x, "x")
    axis = axis % x.dim()
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    if group_size <= 0 or x.shape[axis] % group_size:
        raise ValueError("shape[axis] must be a multiple of group_size")
    q, s, z = _outputs(x, code, _scale_shape(x.shape, axis, group_size), symmetric)
    shp, nd = _shape(x.shape)
    _call("tq_quant_per_group", _ptr(x), _ft(x), nd, shp, axis, group_size, CODE[code], qmin, qmax, _ptr(q),
          _ptr(s), _ptr(z), _stream(x.device))
    return q, s, z


# ------------------------------------------------------------ integer dequantize
def _float_out(shape, dtype, device):
    return torch.empty(tuple(shape), dtype=dtype, device=device)


def tq_dequant_per_tensor(q, shape, scale, zero_point=None, code="s8", out_dtype=torch.float32):
    y = _float_out(shape, out_dtype, q.device)
    _call("tq_dequant_per_tensor", _ptr(q.contiguous()), CODE[code], y.numel(), _ptr(scale), _ptr(zero_point),
          _ptr(y), FTYPE[out_dtype], _stream(q.device))
    return y


def tq_dequant_per_channel(q, shape, scale, zero_point=None, axis=0, code="s8", out_dtype=torch.float32):
    y = _float_out(shape, out_dtype, q.device)
    shp, nd = _shape(shape)
    _call("tq_dequant_per_channel", _ptr(q.contiguous()), CODE[code], nd, shp, axis, _ptr(scale),
          _ptr(zero_point), _ptr(y), FTYPE[out_dtype], _stream(q.device))
    return y


def tq_dequant_per_token(q, shape, scale, zero_point=None, code="s8", out_dtype=torch.float32):
    y = _float_out(shape, out_dtype, q.device)
    cols = shape[-1]
    rows = y.numel() // cols if cols else 0
    _call("tq_dequant_per_token", _ptr(q.contiguous()), CODE[code], rows, cols, _ptr(scale), _ptr(zero_point),
          _ptr(y), FTYPE[out_dtype], _stream(q.device))
    return y


def tq_dequant_per_group(q, shape, scale, zero_point=None, axis=-1, group_size=128, code="u4",
                         out_dtype=torch.float32):
    y = _float_out(shape, out_dtype, q.device)
    axis = axis % len(shape)
    shp, nd = _shape(shape)
    _call("tq_dequant_per_group", _ptr(q.contiguous()), CODE[code], nd, shp, axis, group_size, _ptr(scale),
          _ptr(zero_point), _ptr(y), FTYPE[out_dtype], _stream(q.device))
    return y


# ------------------------------------------------------------ STE backward
def _ste_prep(x, dy):
    x = _dev_float(x, "x")
    dy = _dev_float(dy, "dy")
    if dy.dtype != x.dtype or dy.shape != x.shape:
        raise ValueError("dy must have x's dtype and shape")
    return x, dy, torch.empty_like(x)


def tq_quant_per_tensor_backward(x, dy, scale, zero_point=None, code="s8", qmin=None, qmax=None):
    x, dy, dx = _ste_prep(x, dy)
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    _call("tq_quant_per_tensor_backward", _ptr(x), _ft(x), x.numel(), CODE[code], qmin, qmax, _ptr(scale),
          _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_quant_per_channel_backward(x, dy, scale, zero_point=None, axis=0, code="s8", qmin=None, qmax=None):
    x, dy, dx = _ste_prep(x, dy)
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    shp, nd = _shape(x.shape)
    _call("tq_quant_per_channel_backward", _ptr(x), _ft(x), nd, shp, axis, CODE[code], qmin, qmax, _ptr(scale),
          _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_quant_per_token_backward(x, dy, scale, zero_point=None, code="s8", qmin=None, qmax=None):
    x, dy, dx = _ste_prep(x, dy)
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    _call("tq_quant_per_token_backward", _ptr(x), _ft(x), rows, cols, CODE[code], qmin, qmax, _ptr(scale),
          _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_quant_per_group_backward(x, dy, scale, zero_point=None, axis=-1, group_size=128, code="u4", qmin=None,
                                qmax=None):
    x, dy, dx = _ste_prep(x, dy)
    axis = axis % x.dim()
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    shp, nd = _shape(x.shape)
    _call("tq_quant_per_group_backward", _ptr(x), _ft(x), nd, shp, axis, group_size, CODE[code], qmin, qmax,
          _ptr(scale), _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


# ------------------------------------------------------------ dequant backward
def tq_dequant_per_tensor_backward(dy, scale):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    _call("tq_dequant_per_tensor_backward", _ptr(dy), _ft(dy), dy.numel(), _ptr(scale), _ptr(dq),
          _stream(dy.device))
    return dq


def tq_dequant_per_channel_backward(dy, scale, axis=0):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    shp, nd = _shape(dy.shape)
    _call("tq_dequant_per_channel_backward", _ptr(dy), _ft(dy), nd, shp, axis, _ptr(scale), _ptr(dq),
          _stream(dy.device))
    return dq


def tq_dequant_per_token_backward(dy, scale):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    cols = dy.shape[-1]
    rows = dy.numel() // cols if cols else 0
    _call("tq_dequant_per_token_backward", _ptr(dy), _ft(dy), rows, cols, _ptr(scale), _ptr(dq),
          _stream(dy.device))
    return dq


def tq_dequant_per_group_backward(dy, scale, axis=-1, group_size=128):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    axis = axis % dy.dim()
    shp, nd = _shape(dy.shape)
    _call("tq_dequant_per_group_backward", _ptr(dy), _ft(dy), nd, shp, axis, group_size, _ptr(scale), _ptr(dq),
          _stream(dy.device))
    return dq


# ------------------------------------------------------------ FP8 blocks
def tq_quant_fp8_block(x, block_rows=1, block_cols=128):
    x = _dev_float(x, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((-(-rows // block_rows), -(-cols // block_cols)), dtype=torch.float32, device=x.device)
    _call("tq_quant_fp8_block", _ptr(x), _ft(x), rows, cols, block_rows, block_cols, _ptr(q), _ptr(s),
          _stream(x.device))
    return q, s


def tq_dequant_fp8_block(q, scale, block_rows=1, block_cols=128, out_dtype=torch.bfloat16):
    rows, cols = q.shape
    y = torch.empty((rows, cols), dtype=out_dtype, device=q.device)
    _call("tq_dequant_fp8_block", _ptr(q.contiguous()), rows, cols, block_rows, block_cols, _ptr(scale), _ptr(y),
          FTYPE[out_dtype], _stream(q.device))
    return y


def tq_quant_fp8_block_backward(x, dy, scale, block_rows=1, block_cols=128):
    x, dy, dx = _ste_prep(x, dy)
    rows, cols = x.shape
    _call("tq_quant_fp8_block_backward", _ptr(x), _ft(x), rows, cols, block_rows, block_cols, _ptr(scale),
          _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_dequant_fp8_block_backward(dy, scale, block_rows=1, block_cols=128):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    rows, cols = dy.shape
    _call("tq_dequant_fp8_block_backward", _ptr(dy), _ft(dy), rows, cols, block_rows, block_cols, _ptr(scale),
          _ptr(dq), _stream(dy.device))
    return dq


# ------------------------------------------------------------ FP4 blocks
def tq_quant_fp4_block(x, kind="nvfp4", global_scale=None):
    """Returns (packed [rows, k/2] u8, block scales [rows, k/gs] u8, global
    scale float32[1] for NVFP4 (None for MXFP4)).  Passing ``global_scale``
    makes the NVFP4 per-tensor scale a static input."""
    x = _dev_float(x, "x")
    rows, k = x.shape
    gs = FP4_GROUP[kind]
    packed = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    bs = torch.empty((rows, k // gs), dtype=torch.uint8, device=x.device)
    static = global_scale is not None
    sg = None
    if kind == "nvfp4":
        sg = (global_scale.to(device=x.device, dtype=torch.float32).reshape(1).clone() if static
              else torch.empty(1, dtype=torch.float32, device=x.device))
    ws = torch.empty(max(1, tq_workspace_bytes(1, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_quant_fp4_block", _ptr(x), _ft(x), rows, k, FP4_KIND[kind], _ptr(packed), _ptr(bs), _ptr(sg),
          int(static), _ptr(ws), ws.numel(), _stream(x.device))
    return packed, bs, sg


def tq_quant_fp4_block_noalloc(x, packed, block_scale, global_scale=None, kind="nvfp4", static_global=False):
    """tq_quant_fp4_block into caller-provided outputs, with no workspace and
    no allocation in the library (packed [rows, k/2] u8, block_scale
    [rows, k/gs] u8, global_scale float32[1] for NVFP4: an input when
    static_global, else written)."""
    x = _dev_float(x, "x")
    rows, k = x.shape
    _call("tq_quant_fp4_block_noalloc", _ptr(x), _ft(x), rows, k, FP4_KIND[kind], _ptr(packed), _ptr(block_scale),
          _ptr(global_scale), int(bool(static_global)), _stream(x.device))
    return packed, block_scale, global_scale


def tq_dequant_fp4_block(packed, block_scale, global_scale=None, kind="nvfp4", out_dtype=torch.bfloat16):
    rows, kb = packed.shape
    y = torch.empty((rows, kb * 2), dtype=out_dtype, device=packed.device)
    _call("tq_dequant_fp4_block", _ptr(packed.contiguous()), _ptr(block_scale.contiguous()), _ptr(global_scale),
          rows, kb * 2, FP4_KIND[kind], _ptr(y), FTYPE[out_dtype], _stream(packed.device))
    return y


def tq_quant_fp4_block_backward(x, dy, block_scale, global_scale=None, kind="nvfp4"):
    x, dy, dx = _ste_prep(x, dy)
    rows, k = x.shape
    _call("tq_quant_fp4_block_backward", _ptr(x), _ft(x), _ptr(block_scale.contiguous()), _ptr(global_scale),
          rows, k, FP4_KIND[kind], _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_dequant_fp4_block_backward(dy, block_scale, global_scale=None, kind="nvfp4"):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    rows, k = dy.shape
    _call("tq_dequant_fp4_block_backward", _ptr(dy), _ft(dy), _ptr(block_scale.contiguous()), _ptr(global_scale),
          rows, k, FP4_KIND[kind], _ptr(dq), _stream(dy.device))
    return dq


def tq_fp4_transpose_for_gemm(packed, block_scale, n, k, group_size):
    """packed [n, k/2] -> [k/2, n]; block_scale [n, k/gs] -> [k/gs, n]."""
    pt = torch.empty((k // 2, n), dtype=torch.uint8, device=packed.device)
    st = None if block_scale is None else torch.empty((k // group_size, n), dtype=torch.uint8,
                                                        device=packed.device)
    _call("tq_fp4_transpose_for_gemm", _ptr(packed.contiguous()),
          None if block_scale is None else _ptr(block_scale.contiguous()), n, k, group_size, _ptr(pt), _ptr(st),
          _stream(packed.device))
    return pt, st


def tq_fp4_transpose_concat_for_gemm(parts, k, group_size, align=1):
    """parts: [(packed [n_i, k/2], block_scale [n_i, k/gs] or None), ...].
    Returns (packed_t [k/2, stride], block_scale_t [k/gs, stride] or None,
    stride) with stride = sum(n_i) rounded up to a multiple of ``align``."""
    if not parts:
        raise TQError("tq_fp4_transpose_concat_for_gemm", TQ_ERR_INVALID)
    dev = parts[0][0].device
    packed = [p.contiguous() for p, _ in parts]
    with_scales = all(b is not None for _, b in parts)
    scales = [b.contiguous() for _, b in parts] if with_scales else None
    n = [int(p.shape[0]) for p in packed]
    stride = -(-sum(n) // align) * align if align > 0 else 0
    pt = torch.empty((k // 2, stride), dtype=torch.uint8, device=dev)
    st = torch.empty((k // group_size, stride), dtype=torch.uint8, device=dev) if with_scales else None
    pp = (_P * len(packed))(*[p.data_ptr() for p in packed])
    bb = (_P * len(packed))(*[b.data_ptr() for b in scales]) if with_scales else None
    got = _I64(0)
    _call("tq_fp4_transpose_concat_for_gemm", len(packed), pp, bb, (_I64 * len(n))(*n), k, group_size, align, _ptr(pt),
          _ptr(st), ctypes.byref(got), _stream(dev))
    assert got.value == stride
    return pt, st, stride


def tq_fp4_concat_rows(packed1, block_scale1, global_scale1, packed2, block_scale2, global_scale2, k):
    """Stack two NVFP4 weights by rows; the per-tensor scales are host floats
    that must be bit-identical."""
    n1, n2 = int(packed1.shape[0]), int(packed2.shape[0])
    dev = packed1.device
    po = torch.empty((n1 + n2, k // 2), dtype=torch.uint8, device=dev)
    so = torch.empty((n1 + n2, k // 16), dtype=torch.uint8, device=dev)
    _call("tq_fp4_concat_rows", _ptr(packed1.contiguous()), _ptr(block_scale1.contiguous()), float(global_scale1),
          _ptr(packed2.contiguous()), _ptr(block_scale2.contiguous()), float(global_scale2), n1, n2, k, _ptr(po),
          _ptr(so), _stream(dev))
    return po, so


def tq_fp4_predequant_to_fp8(packed, block_scale, global_scale=1.0, kind="nvfp4"):
    """packed [rows, k/2] -> E4M3 bytes [rows, k] (uint8) with the per-tensor
    scale (a host float) applied."""
    rows, kb = packed.shape
    out = torch.empty((rows, kb * 2), dtype=torch.uint8, device=packed.device)
    _call("tq_fp4_predequant_to_fp8", _ptr(packed.contiguous()), _ptr(block_scale.contiguous()), float(global_scale),
          rows, kb * 2, FP4_KIND[kind], _ptr(out), _stream(packed.device))
    return out


# ------------------------------------------------------------ fake quantization / dynamic range
def tq_fake_quant_per_tensor(x, code="s8", qmin=None, qmax=None, symmetric=True, scale=None, zero_point=None):
    """Per-tensor round trip y = (q - zp) * scale in x's dtype.  Returns
    (y, scale float32[1], zero_point[1] or None); passing ``scale`` (and
    ``zero_point``) makes them static inputs."""
    x = _dev_float(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    static = scale is not None
    s = torch.empty(1, dtype=torch.float32, device=x.device)
    z = None if symmetric else torch.empty(1, dtype=_zp_dtype(code), device=x.device)
    if static:
        s = scale.to(device=x.device, dtype=torch.float32).reshape(1).contiguous()
        if not symmetric:
            z = zero_point.to(device=x.device, dtype=_zp_dtype(code)).reshape(1).contiguous()
    y = torch.empty_like(x)
    ws = torch.empty(max(1, tq_workspace_bytes(0, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_fake_quant_per_tensor", _ptr(x), _ft(x), x.numel(), CODE[code], qmin, qmax, int(static), _ptr(y),
          _ptr(s), _ptr(z), _ptr(ws), ws.numel(), _stream(x.device))
    return y, s, z


def tq_fake_quant_per_tensor_backward(x, dy, scale, zero_point=None, code="s8", qmin=None, qmax=None):
    x, dy, dx = _ste_prep(x, dy)
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    _call("tq_fake_quant_per_tensor_backward", _ptr(x), _ft(x), x.numel(), CODE[code], qmin, qmax, _ptr(scale),
          _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


RANGE_MODE = {"symmetric": 0, "asymmetric": 1}
RANGE_SCOPE = {"tensor": 0, "token": 1, "channel": 2}


def tq_dynamic_range_quantize(x, mode="symmetric", scope="token", code="s8", axis=0):
    """Quantize with the range taken from the data at ``scope`` ('tensor',
    'token' or 'channel' along ``axis``) and the code's default range for
    ``mode``.  Returns (q, scale, zero_point or None)."""
    x = _dev_float(x, "x")
    sym = mode == "symmetric"
    if scope == "tensor":
        sshape = (1,)
    elif scope == "token":
        sshape = (x.numel() // x.shape[-1] if x.shape[-1] else 0,)
    else:
        sshape = (x.shape[axis],)
    q, s, z = _outputs(x, code, sshape, sym)
    shp, nd = _shape(x.shape)
    ws = torch.empty(max(1, tq_workspace_bytes(0, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_dynamic_range_quantize", _ptr(x), _ft(x), nd, shp, RANGE_MODE[mode], RANGE_SCOPE[scope], axis,
          CODE[code], _ptr(q), _ptr(s), _ptr(z), _ptr(ws), ws.numel(), _stream(x.device))
    return q, s, z


# ------------------------------------------------------------ MXFP8
def tq_quant_mxfp8(x):
    """Returns (q [rows, k] E4M3 bytes as uint8, block scales [rows, k/32]
    E8M0 bytes)."""
    x = _dev_float(x, "x")
    rows, k = x.shape
    q = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    bs = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device)
    _call("tq_quant_mxfp8", _ptr(x), _ft(x), rows, k, _ptr(q), _ptr(bs), _stream(x.device))
    return q, bs


def tq_dequant_mxfp8(q, block_scale, out_dtype=torch.bfloat16):
    rows, k = q.shape
    y = torch.empty((rows, k), dtype=out_dtype, device=q.device)
    _call("tq_dequant_mxfp8", _ptr(q.contiguous()), _ptr(block_scale.contiguous()), rows, k, _ptr(y),
          FTYPE[out_dtype], _stream(q.device))
    return y


def tq_quant_mxfp8_backward(x, dy, block_scale):
    x, dy, dx = _ste_prep(x, dy)
    rows, k = x.shape
    _call("tq_quant_mxfp8_backward", _ptr(x), _ft(x), _ptr(block_scale.contiguous()), rows, k, _ptr(dy), _ptr(dx),
          _stream(x.device))
    return dx


def tq_dequant_mxfp8_backward(dy, block_scale):
    dy = _dev_float(dy, "dy")
    dq = torch.empty_like(dy)
    rows, k = dy.shape
    _call("tq_dequant_mxfp8_backward", _ptr(dy), _ft(dy), _ptr(block_scale.contiguous()), rows, k, _ptr(dq),
          _stream(dy.device))
    return dq


# ------------------------------------------------------------ FP8 per tensor
def tq_quant_fp8_per_tensor(x, scale=None):
    """Returns (q E4M3 bytes of x's shape as uint8, scale float32[1]);
    passing ``scale`` makes it a static input."""
    x = _dev_float(x, "x")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    static = scale is not None
    s = (scale.to(device=x.device, dtype=torch.float32).reshape(1).clone() if static
         else torch.empty(1, dtype=torch.float32, device=x.device))
    ws = torch.empty(max(1, tq_workspace_bytes(2, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_quant_fp8_per_tensor", _ptr(x), _ft(x), x.numel(), int(static), _ptr(q), _ptr(s), _ptr(ws),
          ws.numel(), _stream(x.device))
    return q, s


def tq_dequant_fp8_per_tensor(q, scale, out_dtype=torch.bfloat16):
    y = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _call("tq_dequant_fp8_per_tensor", _ptr(q.contiguous()), q.numel(), _ptr(scale), _ptr(y), FTYPE[out_dtype],
          _stream(q.device))
    return y


# ------------------------------------------------------------ binary64 inputs
GRAN = {"tensor": 0, "channel": 1, "token": 2, "group": 3}


def _f64_scale_shape(shape, gran, axis, group_size):
    if gran == "tensor":
        return (1,)
    if gran == "token":
        rows = 1
        for d in shape[:-1]:
            rows *= int(d)
        return (rows,)
    if gran == "channel":
        return (shape[axis],)
    return _scale_shape(shape, axis, group_size)


def _f64(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float64:
        raise TypeError("%s must be a float64 CUDA (HIP) tensor" % name)
    return t.contiguous()


def tq_quant_f64(x, gran="token", axis=0, group_size=0, code="s8", qmin=None, qmax=None, symmetric=True,
                 scale=None, zero_point=None):
    """Binary64 quantize; returns (q, scale float64, zero_point or None)."""
    x = _f64(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    sshape = _f64_scale_shape(tuple(x.shape), gran, axis, group_size)
    q = torch.empty(_packed_shape(x.shape, code), dtype=torch.uint8, device=x.device)
    static = scale is not None
    s = (scale.to(device=x.device, dtype=torch.float64).reshape(sshape).contiguous() if static
         else torch.empty(sshape, dtype=torch.float64, device=x.device))
    z = None
    if not symmetric:
        z = (zero_point.to(device=x.device, dtype=_zp_dtype(code)).reshape(sshape).contiguous() if static
             else torch.empty(sshape, dtype=_zp_dtype(code), device=x.device))
    shp, nd = _shape(x.shape)
    ws = torch.empty(max(1, tq_workspace_bytes(3, x.numel())), dtype=torch.uint8, device=x.device)
    _call("tq_quant_f64", _ptr(x), nd, shp, GRAN[gran], axis, group_size, CODE[code], qmin, qmax, int(static),
          _ptr(q), _ptr(s), _ptr(z), _ptr(ws), ws.numel(), _stream(x.device))
    return q, s, z


def tq_dequant_f64(q, shape, scale, zero_point=None, gran="token", axis=0, group_size=0, code="s8"):
    y = torch.empty(tuple(shape), dtype=torch.float64, device=q.device)
    shp, nd = _shape(shape)
    _call("tq_dequant_f64", _ptr(q.contiguous()), CODE[code], nd, shp, GRAN[gran], axis, group_size, _ptr(scale),
          _ptr(zero_point), _ptr(y), _stream(q.device))
    return y


def tq_quant_f64_backward(x, dy, scale, zero_point=None, gran="token", axis=0, group_size=0, code="s8", qmin=None,
                          qmax=None):
    x, dy = _f64(x, "x"), _f64(dy, "dy")
    qmin, qmax = _range(code, qmin, qmax, zero_point is None)
    dx = torch.empty_like(x)
    shp, nd = _shape(x.shape)
    _call("tq_quant_f64_backward", _ptr(x), nd, shp, GRAN[gran], axis, group_size, CODE[code], qmin, qmax,
          _ptr(scale), _ptr(zero_point), _ptr(dy), _ptr(dx), _stream(x.device))
    return dx


def tq_dequant_f64_backward(dy, scale, gran="token", axis=0, group_size=0):
    dy = _f64(dy, "dy")
    dq = torch.empty_like(dy)
    shp, nd = _shape(dy.shape)
    _call("tq_dequant_f64_backward", _ptr(dy), nd, shp, GRAN[gran], axis, group_size, _ptr(scale), _ptr(dq),
          _stream(dy.device))
    return dq


# ------------------------------------------------------------ row-strided inputs
def _row_strided(x, name):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise TypeError("%s must be a 2-D CUDA (HIP) tensor with unit column stride" % name)
    _ft(x)
    return x


def tq_quant_per_token_strided(x, code="s8", qmin=None, qmax=None, symmetric=True):
    """Per-token quantize of a 2-D view whose rows are strided (e.g. a column
    slice); the view is read in place."""
    x = _row_strided(x, "x")
    qmin, qmax = _range(code, qmin, qmax, symmetric)
    rows, cols = x.shape
    q, s, z = _outputs(x, code, (rows,), symmetric)
    _call("tq_quant_per_token_strided", _ptr(x), _ft(x), rows, cols, x.stride(0), CODE[code], qmin, qmax, _ptr(q),
          _ptr(s), _ptr(z), _stream(x.device))
    return q, s, z


def tq_quant_fp8_rows_strided(x, block_cols=128):
    x = _row_strided(x, "x")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, cols // block_cols), dtype=torch.float32, device=x.device)
    _call("tq_quant_fp8_rows_strided", _ptr(x), _ft(x), rows, cols, x.stride(0), block_cols, _ptr(q), _ptr(s),
          _stream(x.device))
    return q, s


# ------------------------------------------------------------ FP8 block GEMM
def tq_fp8_block_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16):
    """y = x W^T from E4M3 activations qa [M, K] (scales sa [M, K/128]) and
    E4M3 weights qw [N, K] (scales sw [N/128, K/128])."""
    M, K = qa.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=qa.device)
    _call("tq_fp8_block_gemm", _ptr(qa.contiguous()), _ptr(sa.contiguous()), _ptr(qw.contiguous()),
          _ptr(sw.contiguous()), M, N, K, _ptr(y), FTYPE[out_dtype], _stream(qa.device))
    return y


# ------------------------------------------------------- W8A8 quantized linear
def tq_w8a8_linear(qx, sx, qw, sw, out_dtype=torch.bfloat16):
    """y = x W^T from s8 activation codes qx [M, K] (per-row scales sx [M])
    and s8 weight codes qw [N, K] (per-channel scales sw [N])."""
    M, K = qx.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=qx.device)
    _call("tq_w8a8_linear", _ptr(qx.contiguous()), _ptr(sx.contiguous()), _ptr(qw.contiguous()),
          _ptr(sw.contiguous()), M, N, K, _ptr(y), FTYPE[out_dtype], _stream(qx.device))
    return y


# ------------------------------------------------------ FP4 weight-only linear
def tq_fp4_linear(x, packed, block_scale, global_scale, kind="nvfp4", out_dtype=torch.bfloat16):
    """y = x W^T from bf16 activations x [M, K] and an FP4 weight in the
    quantizer's layout (packed [N, K/2], block scales [N, K/gs], NVFP4
    per-tensor scale as a one-element device tensor)."""
    M, K = x.shape
    N = packed.shape[0]
    y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _call("tq_fp4_linear", _ptr(x.contiguous()), FTYPE[x.dtype], _ptr(packed.contiguous()), _ptr(block_scale.contiguous()),
          _ptr(global_scale) if global_scale is not None else None, FP4_KIND[kind], M, N, K, _ptr(y), FTYPE[out_dtype],
          _stream(x.device))
    return y
