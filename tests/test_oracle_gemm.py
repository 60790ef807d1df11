"""Pins of the oracle's FP8 block GEMM (smile.llm.quant Fp8BlockGemm: 1 x 128
activation scales, 128 x 128 weight scales, out = x W^T).

Checked against numpy's float64 matmul of matrices dequantized
independently (E4M3 values from the format's enumeration, scales expanded
with np.repeat), which fixes the operand orientation, the block indexing of
both scale arrays and the summation structure; and against exact integer
results when every value, product and scale is exactly representable."""
import numpy as np
import pytest

import bruteforce as bf
import workloads


def _dec_table():
    mags = bf.e4m3_magnitudes()
    dec = np.zeros(256)
    dec[:127], dec[128:255] = mags, -mags
    dec[127] = dec[255] = np.nan
    return dec


def _quant(orc, shape, block, seed, sigma=1.0):
    x = workloads.normal(shape, sigma, seed, "bf16")
    return orc.quant_fp8_block(x, "bf16", *block)


@pytest.mark.parametrize("M,N,K", [(16, 128, 256), (5, 256, 384), (128, 128, 128)])
def test_gemm_matches_numpy_of_dequantized(orc, M, N, K):
    qa, sa = _quant(orc, (M, K), (1, 128), M + K)
    qw, sw = _quant(orc, (N, K), (128, 128), N + K + 1, 0.02)
    y, ya = orc.fp8_block_gemm(qa, sa, qw, sw)
    dec = _dec_table()
    A = dec[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    W = dec[qw] * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)
    ref = A @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * ya + 1e-300)
    assert np.all(ya >= np.abs(y) * (1 - 1e-12))


def test_gemm_exact_integers(orc):
    rng = np.random.default_rng(3)
    M, N, K = 8, 128, 256
    vals = np.array([0.0, 1.0, -1.0, 2.0, -2.0, 0.5])
    codes = orc.enc_e4m3(vals.astype(np.float32))
    ia = rng.integers(0, len(vals), (M, K))
    iw = rng.integers(0, len(vals), (N, K))
    qa, qw = codes[ia], codes[iw]
    sa = np.float32(2.0) ** rng.integers(-3, 4, (M, K // 128)).astype(np.float32)
    sw = np.float32(2.0) ** rng.integers(-3, 4, (N // 128, K // 128)).astype(np.float32)
    y, _ = orc.fp8_block_gemm(qa, sa, qw, sw)
    want = np.zeros((M, N))
    for kb in range(K // 128):
        blk = vals[ia[:, kb * 128:(kb + 1) * 128]] @ vals[iw[:, kb * 128:(kb + 1) * 128]].T
        want += blk * sa[:, kb:kb + 1] * np.repeat(sw[:, kb], 128)[None, :]
    assert (y == want).all()


def test_gemm_rejects_ragged(orc):
    with pytest.raises(ValueError):
        orc.fp8_block_gemm(np.zeros((2, 100), np.uint8), np.zeros((2, 1), np.float32), np.zeros((128, 100), np.uint8),
                           np.zeros((1, 1), np.float32))
