"""Pins of the oracle's FP4 weight-only linear (metrale QuantizedWeight: the
packed E2M1 weight with block scales and a per-tensor scale, made for a
16-bit-activation tile GEMM; smile.llm.quant Nvfp4Linear).  y = x W^T with W
the dequantized weight, evaluated in binary64."""
import numpy as np

import oracle as orc
import workloads


def f32_to_bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)   # exact for bf16 values


def bits_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_hand_example_nvfp4():
    # K = 16: one NVFP4 group; codes 0..15 of row 0 in order (low nibble first),
    # block scale byte 0x38 (1.0), per-tensor scale 0.5; x = 1 everywhere
    e2m1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    packed = np.array([[c | ((c + 1) << 4) for c in range(0, 16, 2)]], np.uint8)
    x = f32_to_bf16_bits(np.ones((1, 16), np.float32))
    y, yabs = orc.fp4_linear(x, packed, np.array([[0x38]], np.uint8), 0.5, "nvfp4")
    assert y[0, 0] == 0.5 * sum(e2m1) == 0.0
    assert yabs[0, 0] == 0.5 * sum(abs(v) for v in e2m1) == 18.0


def test_nibble_order():
    # only k = 2 (low nibble of byte 1) holds a code: x[2] alone must show up
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 1] = 0x02                       # E2M1 code 2 = 1.0 at k = 2
    x = np.zeros((1, 32), np.float32)
    x[0, 2], x[0, 3] = 3.0, 5.0
    y, _ = orc.fp4_linear(f32_to_bf16_bits(x), packed, np.full((1, 1), 127, np.uint8), 1.0, "mxfp4")
    assert y[0, 0] == 3.0


def _weights(kind, n, k, seed):
    w = workloads.normal((n, k), 0.02, seed, "bf16")
    return orc.quant_fp4_block(w, "bf16", kind)


def test_matches_dequantized_matmul():
    # the same product through the dequantize (pinned exactly in test_oracle_fp_backward.py) and a float64 matmul
    for kind in ("nvfp4", "mxfp4"):
        packed, bs, sg = _weights(kind, 24, 128, 11)
        x = workloads.normal((5, 128), 1.0, 12, "bf16")
        y, yabs = orc.fp4_linear(x, packed, bs, sg, kind)
        W = orc.dequant_fp4_block(packed, bs, sg, kind, "f32").astype(np.float64)
        ref = bits_to_f64(x) @ W.T
        # NVFP4's dequantize rounds val(scale) * s_g to binary32 first: 2^-24 per element
        tol = (2.0 ** -23 if kind == "nvfp4" else 2.0 ** -50) * yabs
        assert np.all(np.abs(y - ref) <= tol), kind
        assert np.all(yabs >= np.abs(y))


def test_mxfp4_integer_case_is_exact():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (6, 64))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    bs = np.full((6, 2), 128, np.uint8)       # 2^1
    xv = rng.integers(-8, 9, (3, 64)).astype(np.float32)
    y, _ = orc.fp4_linear(f32_to_bf16_bits(xv), packed, bs, 1.0, "mxfp4")
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0, -0.5, -1, -1.5, -2, -3, -4, -6])
    assert np.array_equal(y, xv.astype(np.float64) @ (2.0 * e2m1[codes]).T)
