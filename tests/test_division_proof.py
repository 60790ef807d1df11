"""The one-correction FMA division used by the quantize kernels for bf16 and
f16 inputs equals IEEE binary32 division: exhaustive over all dividend
significands of the input type and all binary32 divisor significands
(2^30 and 2^33 pairs), on the host's IEEE FMA.  CPU only."""
import os
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "proofs")


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("proof") / "division_exhaustive")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-o", exe,
                           os.path.join(HERE, "division_exhaustive.c"), "-lm"])
    return exe


@pytest.mark.parametrize("fbits", [7, 10])
def test_one_correction_division_is_exact(prog, fbits):
    out = subprocess.run([prog, str(fbits)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert " 0 mismatches" in out.stdout


def test_two_correction_binary64_division(tmp_path):
    """The binary64 quantize kernels divide by x * RN(1/s) with two FMA
    corrections: equal to IEEE a / b on 4M random pairs and 1.5M pairs whose
    quotient lies within 2^-105 of a midpoint between binary64 numbers."""
    exe = str(tmp_path / "division_f64")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "division_f64.c"), "-lm"])
    out = subprocess.run([exe, "2000000"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "two corrections: 0 mismatches" in out.stdout


def test_two_correction_binary32_division(tmp_path):
    """Binary32 dividends (f32 inputs, the asymmetric range mx - mn) take two
    FMA corrections of x * RN(1/s): equal to IEEE x / s on 8M random pairs
    over the guarded range 2^-40 <= |s| <= 2^40, 2^-78 <= |x| <= 2^86 (half of
    them with |x / s| <= 255, the code range) and on about 3M pairs whose
    quotient lies within 15 * 2^-48 of a midpoint between binary32 numbers."""
    exe = str(tmp_path / "division_f32")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "division_f32.c"),
                           "-lm"])
    out = subprocess.run([exe, "4000000"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "two corrections: 0 mismatches" in out.stdout
    hard = int(out.stdout.split(" near-midpoint pairs")[0].split("\n")[-1])
    assert hard > 2_000_000
