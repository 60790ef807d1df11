"""The matrix-core arithmetic that the consumer GEMMs' error bounds rest on,
checked on the GPU against exact sums (tests/proofs/mfma_probe.hip, built by
__graft_entry__.build()): one E4M3 x E4M3 16x16x128 step stays within the
per-step bound the FP8 GEMM test uses (intra-group truncation granules plus
(17 * 2^-21 + 2^-23) of the magnitude sum), on random codes over the whole
E4M3 range and on a narrow exponent window; one bf16 x bf16 16x16x32 step
stays within 33 units of 2^(E-24) (E: exponent of the largest product), the
FP4 linear's per-step allowance; s8 x s8 16x16x64 steps are exact."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "proofs", "mfma_probe")


def test_matrix_core_steps_within_the_gemm_bounds():
    assert os.path.exists(EXE), "build the probe with __graft_entry__.build()"
    print("running", EXE, flush=True)
    out = subprocess.run([EXE, "4096"], capture_output=True, text=True, timeout=120)
    print(out.stdout, flush=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "RESULT: every error within its bound" in out.stdout
    assert "mismatches 0" in out.stdout
