"""The gfx950 code objects contain no instruction that would break the
binary32 rounding the oracle defines: no packed-FP32 arithmetic (disabled at
build time), no mixed-precision FMA with an f16 result (v_fma_mixlo_f16 /
v_fma_mixhi_f16 / v_mad_mix* round a product once into f16), and no scratch
spills.  v_fma_mix_f32 is allowed: it widens f16 operands exactly and rounds
once to binary32, the same result as the f32 FMA of the widened values.
Compiles each kernel source to AMD assembly on the CPU (hipcc
cross-compiles)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_quantization_amd", "csrc")


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_tq_hipbuild", os.path.join(ROOT, "tensor_quantization_amd",
                                                                                "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _asm(src, tmp):
    b = _build_module()
    out = os.path.join(tmp, os.path.basename(src) + ".s")
    subprocess.check_call([b.HIPCC, *b.FLAGS, "-S", "--cuda-device-only", src, "-o", out],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return open(out).read()


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("isa"))
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(4) as ex:
        return dict(zip(srcs, ex.map(lambda s: _asm(s, tmp), srcs)))


def test_no_packed_fp32_or_mixed_fma(listings):
    for src, text in listings.items():
        bad = re.findall(r"\b(v_pk_(?:fma|mul|add|mov)_f32|v_fma_mix(?:lo|hi)\w*|v_mad_mix\w*)\b", text)
        assert not bad, (os.path.basename(src), sorted(set(bad)))


def test_no_scratch(listings):
    for src, text in listings.items():
        sizes = [int(v) for v in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
        assert max(sizes, default=0) == 0, os.path.basename(src)
