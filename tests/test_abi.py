"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/tq.h declares, and rejects malformed arguments on the host
before anything is enqueued (only calls that fail validation are made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    import tensor_quantization_amd as t
    return t


def _declared():
    text = open(os.path.join(ROOT, "include", "tq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(tq):
    names = _declared()
    assert {"tq_quant_per_token", "tq_quant_fp4_block", "tq_fp4_transpose_for_gemm"} <= set(names)
    for n in names:
        assert hasattr(tq._lib, n), n
    assert sorted(tq.EXPORTED) == names
    for n in names:                      # the binding uses the C names
        assert callable(getattr(tq, n, None)) or n in ("tq_status_str",), n


def test_status_and_version(tq):
    assert tq.tq_abi_version() == 1
    assert tq._lib.tq_status_str(0) == b"ok"
    assert tq._lib.tq_status_str(3) == b"misaligned pointer"


def test_default_ranges_match_oracle(tq, orc):
    for code in ("s8", "u8", "s4", "u4"):
        for sym in (True, False):
            if code in ("u8", "u4") and sym:
                with pytest.raises(tq.TQError):
                    tq.tq_default_q_range(code, sym)
                continue
            assert tq.tq_default_q_range(code, sym) == orc.default_q_range(code, sym)


P = ctypes.c_void_p
A = P(0x10000)          # aligned fake device addresses: never dereferenced,
B = P(0x20000)          # every call below fails validation first
C = P(0x30000)
MIS = P(0x10008)


def _shape(*s):
    return (ctypes.c_int64 * len(s))(*s), len(s)


def test_integer_validation(tq):
    L = tq._lib
    INV, ALIGN = tq.TQ_ERR_INVALID, tq.TQ_ERR_ALIGN
    # null pointers, bad dtype, bad ranges
    assert L.tq_quant_per_token(None, 2, 4, 8, 0, -127, 127, B, C, None, None) == INV
    assert L.tq_quant_per_token(A, 7, 4, 8, 0, -127, 127, B, C, None, None) == INV
    assert L.tq_quant_per_token(A, 2, 4, 8, 0, -128, 127, B, C, None, None) == INV   # symmetric needs -qmax
    assert L.tq_quant_per_token(A, 2, 4, 8, 1, 0, 255, B, C, None, None) == INV      # symmetric unsigned
    assert L.tq_quant_per_token(A, 2, 4, 8, 0, 5, 5, B, C, A, None) == INV           # qmin >= qmax
    assert L.tq_quant_per_token(A, 2, 4, 8, 3, 0, 16, B, C, A, None) == INV          # beyond u4
    assert L.tq_quant_per_token(A, 2, 4, 7, 3, 0, 15, B, C, A, None) == INV          # odd last dim, 4-bit
    assert L.tq_quant_per_token(A, 2, -1, 8, 0, -127, 127, B, C, None, None) == INV
    assert L.tq_quant_per_token(MIS, 2, 4, 8, 0, -127, 127, B, C, None, None) == ALIGN
    # group size must divide the axis; axis in range
    shp, nd = _shape(4, 100)
    assert L.tq_quant_per_group(A, 1, nd, shp, 1, 128, 3, 0, 15, B, C, A, None) == INV
    assert L.tq_quant_per_group(A, 1, nd, shp, 2, 4, 3, 0, 15, B, C, A, None) == INV
    assert L.tq_quant_per_channel(A, 1, nd, shp, -1, 0, -127, 127, B, C, None, None) == INV
    # a large per-tensor dynamic scale needs a workspace (small tensors reduce in one block)
    assert L.tq_quant_per_tensor(A, 0, ctypes.c_int64(1 << 20), 0, -127, 127, 0, B, C, None, None, 0, None) == INV
    assert tq.tq_workspace_bytes(0, 1 << 16) == 0 and tq.tq_workspace_bytes(0, 1 << 20) > 0
    # dequant / STE / dequant-backward
    assert L.tq_dequant_per_token(None, 0, 4, 8, C, None, B, 2, None) == INV
    assert L.tq_dequant_per_token(A, 0, 4, 8, C, None, B, 9, None) == INV
    assert L.tq_dequant_per_token(A, 3, 4, 7, C, None, B, 2, None) == INV
    assert L.tq_quant_per_token_backward(A, 2, 4, 8, 0, -127, 127, C, None, None, B, None) == INV
    assert L.tq_quant_per_token_backward(A, 2, 4, 8, 0, -127, 127, C, None, MIS, B, None) == ALIGN
    assert L.tq_dequant_per_token_backward(A, 2, 4, 8, None, B, None) == INV


def test_fp8_fp4_validation(tq):
    L = tq._lib
    INV, ALIGN = tq.TQ_ERR_INVALID, tq.TQ_ERR_ALIGN
    assert L.tq_quant_fp8_block(A, 2, 128, 128, 0, 128, B, C, None) == INV       # block rows 0
    assert L.tq_quant_fp8_block(A, 2, 128, 128, 1, -128, B, C, None) == INV      # negative block
    assert L.tq_quant_fp8_block(A, 2, -1, 128, 1, 128, B, C, None) == INV
    assert L.tq_quant_fp8_block(A, 7, 128, 128, 1, 128, B, C, None) == INV       # bad dtype
    assert L.tq_quant_fp8_block(MIS, 2, 128, 128, 1, 128, B, C, None) == ALIGN
    assert L.tq_dequant_fp8_block(A, 128, 128, 1, 128, None, B, 2, None) == INV
    assert L.tq_quant_fp4_block(A, 2, 4, 24, 0, B, C, A, 1, None, 0, None) == INV   # k % 16
    assert L.tq_quant_fp4_block(A, 2, 4, 48, 1, B, C, None, 0, None, 0, None) == INV  # k % 32
    assert L.tq_quant_fp4_block(A, 2, 4, 32, 0, B, C, None, 1, None, 0, None) == INV  # NVFP4 needs s_g
    assert L.tq_quant_fp4_block(A, 2, 4, 32, 0, B, C, A, 0, None, 0, None) == INV     # dynamic needs ws
    assert L.tq_quant_fp4_block(A, 2, 4, 32, 5, B, C, A, 1, None, 0, None) == INV     # bad kind
    assert L.tq_dequant_fp4_block(A, B, None, 4, 32, 0, C, 2, None) == INV
    assert L.tq_fp4_transpose_for_gemm(A, B, 4, 31, 16, C, A, None) == INV
    assert L.tq_fp4_transpose_for_gemm(A, B, 4, 32, 16, C, None, None) == INV
    assert L.tq_quant_mxfp8(A, 2, 4, 48, B, C, None) == INV                       # k % 32
    assert L.tq_quant_mxfp8(MIS, 2, 4, 64, B, C, None) == ALIGN
    assert L.tq_dequant_mxfp8(A, None, 4, 64, B, 2, None) == INV


def test_follow_on_validation(tq):
    L = tq._lib
    INV = tq.TQ_ERR_INVALID
    P2 = (ctypes.c_void_p * 2)(A.value, B.value)
    N2 = (ctypes.c_int64 * 2)(16, 16)
    stride = ctypes.c_int64(-1)
    assert L.tq_fp4_transpose_concat_for_gemm(0, P2, P2, N2, 32, 16, 1, C, C, None, None) == INV   # empty list
    assert L.tq_fp4_transpose_concat_for_gemm(2, P2, P2, N2, 32, 16, 0, C, C, None, None) == INV   # align 0
    assert L.tq_fp4_transpose_concat_for_gemm(2, P2, P2, N2, 31, 16, 1, C, C, None, None) == INV   # odd k
    assert L.tq_fp4_transpose_concat_for_gemm(2, P2, P2, N2, 0, 16, 48, C, C, ctypes.byref(stride),
                                              None) == tq.TQ_OK                                   # k = 0: no work
    assert stride.value == 48
    assert L.tq_fp4_concat_rows(A, B, 1.0, A, B, 2.0, 4, 4, 32, C, C, None) == INV     # scales differ
    assert L.tq_fp4_concat_rows(A, B, 0.0, A, B, -0.0, 4, 4, 32, C, C, None) == INV    # +0 vs -0
    assert L.tq_fp4_concat_rows(A, B, 1.0, A, B, 1.0, 4, 4, 24, C, C, None) == INV     # k % 16
    assert L.tq_fp4_predequant_to_fp8(A, B, 1.0, 4, 24, 0, C, None) == INV             # k % 16
    assert L.tq_fp4_predequant_to_fp8(A, B, 1.0, 4, 32, 3, C, None) == INV             # bad kind
    assert L.tq_fake_quant_per_tensor(A, 2, 64, 1, -127, 127, 0, B, C, None, None, 0, None) == INV  # u8 sym
    assert L.tq_fake_quant_per_tensor(A, 2, -1, 0, -127, 127, 0, B, C, None, None, 0, None) == INV
    assert L.tq_fake_quant_per_tensor_backward(A, 2, 64, 0, -127, 127, C, None, None, B, None) == INV  # no dy
    shp = (ctypes.c_int64 * 2)(4, 8)
    assert L.tq_dynamic_range_quantize(A, 2, 2, shp, 2, 1, 0, 0, B, C, None, None, 0, None) == INV  # bad mode
    assert L.tq_dynamic_range_quantize(A, 2, 2, shp, 0, 3, 0, 0, B, C, None, None, 0, None) == INV  # bad scope
    assert L.tq_dynamic_range_quantize(A, 2, 2, shp, 0, 1, 0, 1, B, C, None, None, 0, None) == INV  # u8 sym
    assert L.tq_dynamic_range_quantize(A, 2, 2, shp, 1, 1, 0, 1, B, C, None, None, 0, None) == INV  # no zp
    assert L.tq_dynamic_range_quantize(A, 2, 2, shp, 0, 2, 5, 0, B, C, None, None, 0, None) == INV  # bad axis


def test_gemm_validation(tq):
    L = tq._lib
    INV, UNS, ALIGN = tq.TQ_ERR_INVALID, tq.TQ_ERR_UNSUPPORTED, tq.TQ_ERR_ALIGN
    assert L.tq_fp8_block_gemm(A, C, A, C, 128, 100, 128, B, 2, None) == INV      # N % 128
    assert L.tq_fp8_block_gemm(A, C, A, C, 128, 128, 64, B, 2, None) == INV       # K % 128
    assert L.tq_fp8_block_gemm(A, C, A, C, 128, 128, 128, B, 5, None) == INV      # bad dtype
    assert L.tq_fp8_block_gemm(None, C, A, C, 128, 128, 128, B, 2, None) == INV
    assert L.tq_fp8_block_gemm(MIS, C, A, C, 128, 128, 128, B, 2, None) == ALIGN
    assert L.tq_w8a8_linear(A, C, A, C, 128, 100, 128, B, 2, None) == UNS         # N % 128
    assert L.tq_w8a8_linear(A, C, A, C, 128, 128, 131072, B, 2, None) == UNS      # sums would pass 32 bits
    assert L.tq_w8a8_linear(A, C, A, C, 128, 128, 128, B, 7, None) == INV
    assert L.tq_w8a8_linear(A, None, A, C, 128, 128, 128, B, 2, None) == INV
    assert L.tq_w8a8_linear(A, C, MIS, C, 128, 128, 128, B, 2, None) == ALIGN
    assert L.tq_fp4_linear(A, 2, A, C, C, 0, 128, 100, 64, B, 2, None) == UNS     # N % 128
    assert L.tq_fp4_linear(A, 2, A, C, C, 0, 128, 128, 32, B, 2, None) == UNS     # K % 64
    assert L.tq_fp4_linear(A, 1, A, C, C, 0, 128, 128, 64, B, 2, None) == UNS     # f16 activations
    assert L.tq_fp4_linear(A, 2, A, C, None, 0, 128, 128, 64, B, 2, None) == INV  # NVFP4 needs s_g
    assert L.tq_fp4_linear(A, 2, A, C, C, 4, 128, 128, 64, B, 2, None) == INV     # bad kind
    assert L.tq_fp4_linear(MIS, 2, A, C, C, 1, 128, 128, 64, B, 2, None) == ALIGN
    # outputs are stored four elements at a time: y aligned to 4 elements
    assert L.tq_fp8_block_gemm(A, C, A, C, 128, 128, 128, P(0x20008), 0, None) == ALIGN   # f32 y on 8 bytes
    assert L.tq_w8a8_linear(A, C, A, C, 128, 128, 128, P(0x20004), 2, None) == ALIGN       # bf16 y on 4 bytes
    assert L.tq_fp4_linear(A, 2, A, C, C, 1, 128, 128, 64, P(0x20002), 1, None) == ALIGN   # f16 y on 2 bytes


def test_stream_mix_validation(tq):
    L = tq._lib
    INV, UNS, ALIGN = tq.TQ_ERR_INVALID, tq.TQ_ERR_UNSUPPORTED, tq.TQ_ERR_ALIGN
    assert L.tq_stream_mix(A, B, 0, 16, 8, 1, 1, None) == 0           # nothing to do
    assert L.tq_stream_mix(None, B, 64, 16, 8, 1, 1, None) == INV
    assert L.tq_stream_mix(A, B, -1, 16, 8, 1, 1, None) == INV
    assert L.tq_stream_mix(A, B, 64, 16, 8, 3, 1, None) == INV        # unknown store policy
    assert L.tq_stream_mix(A, B, 64, 16, 8, 1, 3, None) == INV        # 1, 2 or 4 units per lane
    assert L.tq_stream_mix(MIS, B, 64, 16, 8, 1, 1, None) == ALIGN
    assert L.tq_stream_mix(A, B, 64, 16, 8, 2, 1, None) == UNS        # device scope needs 16-byte stores
    assert L.tq_stream_mix(A, B, 64, 2, 8, 0, 1, None) == UNS         # mix not offered


def test_empty_inputs_enqueue_nothing(tq):
    L = tq._lib
    assert L.tq_quant_per_token(A, 2, 0, 8, 0, -127, 127, B, C, None, None) == 0
    assert L.tq_quant_fp8_block(A, 2, 0, 128, 1, 128, B, C, None) == 0
    assert L.tq_quant_fp4_block(A, 2, 0, 32, 1, B, C, None, 0, None, 0, None) == 0
    assert L.tq_fp8_block_gemm(A, C, A, C, 0, 128, 128, B, 2, None) == 0
    assert L.tq_w8a8_linear(A, C, A, C, 5, 0, 128, B, 2, None) == 0


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "tensor_quantization_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, f)
    for f in os.listdir(os.path.join(ROOT, "include")):
        assert "oracle" not in open(os.path.join(ROOT, "include", f)).read().lower()
