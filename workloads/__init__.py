"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds none of the quantization arithmetic: it only draws
numbers.  Every tensor is ``numpy.random.default_rng(seed)`` standard normal
in float32, times sigma, then rounded to nearest even into the storage type
(numpy's float16 cast, torch's CPU bfloat16 cast).  Float tensors are
returned as numpy arrays in storage form: ``float32`` for f32 and ``uint16``
bit patterns for f16 / bf16.

The workloads are the five the method is measured on (shapes, distributions
and seeds as listed below); no public dataset is involved and none is
imitated.
"""
from __future__ import annotations

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}


def to_storage(v32: np.ndarray, ft: str) -> np.ndarray:
    """Round float32 values to the storage type (RNE) and return its bits."""
    v32 = np.ascontiguousarray(v32, np.float32)
    if ft == "f32":
        return v32
    if ft == "f16":
        return v32.astype(np.float16).view(np.uint16)
    import torch  # bfloat16 rounding: torch's CPU cast is round-to-nearest-even
    return torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal(shape, sigma: float, seed: int, ft: str) -> np.ndarray:
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(sigma)
    return to_storage(v, ft)


def outlier_columns(cols: int, frac: float, seed: int) -> np.ndarray:
    """round(frac * cols) distinct column indices chosen by ``seed``."""
    n = int(round(frac * cols))
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(cols, size=n, replace=False))


def normal_with_outlier_columns(shape, sigma, seed, ft, frac, factor, col_seed):
    """N(0, sigma) with the same round(frac*cols) columns in every row
    multiplied by ``factor`` in float32 before rounding to storage."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(sigma)
    cols = outlier_columns(shape[-1], frac, col_seed)
    v[..., cols] *= np.float32(factor)
    return to_storage(v, ft)


# The five workloads.  ``scale_rows`` lets tests and the CPU baseline take a
# leading-row slice of the same distribution (the generator is row-major, so
# the first r rows of a full draw equal a draw of shape [r, K]).
CONFIGS = {
    "c1_per_tensor_s8": dict(shape=(64, 256), dtype="f32", sigma=1.0, seed=101, dy_seed=102),
    "c2_per_token_s8": dict(shape=(8192, 4096), dtype="bf16", sigma=1.0, seed=201, dy_seed=202,
                            outlier_frac=0.01, outlier_factor=20.0, outlier_seed=203),
    "c3_per_group_u4_g128": dict(shape=(11008, 4096), dtype="f16", sigma=0.02, seed=301,
                                 group_size=128),
    "c4_fp8_act_1x128": dict(shape=(4096, 7168), dtype="bf16", sigma=1.0, seed=401, block=(1, 128)),
    "c4_fp8_weight_128x128": dict(shape=(7168, 7168), dtype="bf16", sigma=0.02, seed=402, block=(128, 128)),
    "c5_fp4_weight": dict(shape=(14336, 4096), dtype="bf16", sigma=0.02, seed=501),
}


def make_input(name: str, rows: int | None = None) -> np.ndarray:
    """The input tensor of workload ``name``; ``rows`` keeps the first rows."""
    c = CONFIGS[name]
    shape = tuple(c["shape"])
    if rows is not None:
        shape = (rows,) + shape[1:]
    if "outlier_frac" in c:
        return normal_with_outlier_columns(shape, c["sigma"], c["seed"], c["dtype"],
                                           c["outlier_frac"], c["outlier_factor"], c["outlier_seed"])
    return normal(shape, c["sigma"], c["seed"], c["dtype"])


def make_dy(name: str, rows: int | None = None) -> np.ndarray:
    """Upstream gradient for the backward ops: N(0, 1) in the input's type."""
    c = CONFIGS[name]
    shape = tuple(c["shape"])
    if rows is not None:
        shape = (rows,) + shape[1:]
    return normal(shape, 1.0, c.get("dy_seed", c["seed"] + 1000), c["dtype"])
