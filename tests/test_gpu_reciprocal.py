"""On gfx950, v_rcp_f32 followed by one Newton step equals the IEEE
reciprocal for every binary32 significand at every exponent of the kernels'
fast divisor range [2^-40, 2^40] (81 x 2^23 divisors) -- the per-group
reciprocal the kernels use there.  Runs the probe program that
__graft_entry__.build() compiles (tests/proofs/rcp_probe.hip)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "proofs", "rcp_probe")


def test_rcp_newton_is_correctly_rounded():
    assert os.path.exists(EXE), "build the probe with __graft_entry__.build()"
    print("running", EXE, flush=True)
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "over 81 exponents (-40..40), 679477248 divisors: 0 mismatches" in out.stdout, out.stdout
