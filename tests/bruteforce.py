"""Independent brute-force checkers used to pin the oracle.

Nothing here calls the oracle.  Rounding is done by exhaustive nearest-value
search over a format's value list (ties to the code with an even last
mantissa bit, which for these formats is the code's lowest bit), binary32
steps use numpy float32 arithmetic (IEEE round-to-nearest-even), and value
lists come from the golden fixtures (OCP definitions), not from the oracle's
decoders.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    codes, vals = [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            codes.append(int(c, 16))
            vals.append(float(v))
    return np.array(codes), np.array(vals)


def e2m1_magnitudes():
    codes, vals = read_table("e2m1_values.txt")
    return np.array([vals[list(codes).index(c)] for c in range(8)])


def e4m3_magnitudes():
    """All 127 finite non-negative E4M3FN values in code order, enumerated
    from the format's structure: subnormals k * 2^-9 (k = 0..7), then in each
    binade [2^e, 2^(e+1)), e = -6..8, eight equally spaced values (3 mantissa
    bits); the last pattern of the top binade is NaN, leaving 448 as the
    largest.  The tests check this list against the golden fixed points."""
    vals = [k * 2.0 ** -9 for k in range(8)]          # subnormals (0x00..0x07)
    for e in range(-6, 9):
        for m in range(8):
            vals.append((1 + m / 8) * 2.0 ** e)
    vals = np.array(vals[:127])                         # 0x7F is NaN
    return vals


def nearest_code(v, mags, sign_bit):
    """Round each float32 value in v to the nearest entry of the sorted
    magnitude list ``mags`` (index = code without sign bit), ties to the
    even index, saturating at the largest entry; ``sign_bit`` is set from
    v's sign bit, so -0 and negative tiny values keep their sign.
    Comparisons are exact: 2|v| against lo + hi."""
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    n = len(mags)
    idx = np.searchsorted(mags, a, side="left")         # mags[idx-1] < a <= mags[idx]
    hi = np.clip(idx, 0, n - 1)
    lo = np.clip(idx - 1, 0, n - 1)
    two_a = 2.0 * a
    mid = mags[lo] + mags[hi]
    pick_hi = (two_a > mid) | ((two_a == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= mags[-1], n - 1, code)
    code = np.where(a == 0, 0, code)
    neg = np.signbit(v)
    return (code | np.where(neg, sign_bit, 0)).astype(np.uint8)


def f32(x):
    return np.float32(x)


def div32(a, b):
    """IEEE binary32 division (numpy float32, round to nearest even)."""
    with np.errstate(all="ignore"):
        return np.float32(np.float32(a) / np.float32(b))


def mul32(a, b):
    with np.errstate(all="ignore"):
        return np.float32(np.float32(a) * np.float32(b))


def nearest_int_code(v, qmin, qmax, zp):
    """Nearest code c in [qmin, qmax] to the real value v + zp, measured on
    the grid c - zp; ties to even (c - zp).  Exhaustive over the range."""
    v = float(v)
    best, bd = None, None
    for c in range(qmin, qmax + 1):
        d = abs(v - (c - zp))
        if best is None or d < bd or (d == bd and (c - zp) % 2 == 0):
            best, bd = c, d
    return best
