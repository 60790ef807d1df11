"""The gfx950 code objects contain no instruction that would break the
binary32 rounding the oracle defines: no packed-FP32 arithmetic (disabled at
build time), no mixed-precision FMA with an f16 result (v_fma_mixlo_f16 /
v_fma_mixhi_f16 / v_mad_mix* round a product once into f16), and no scratch
spills.  v_fma_mix_f32 is allowed: it widens f16 operands exactly and rounds
once to binary32, the same result as the f32 FMA of the widened values.

Nor does any 12- or 16-byte global store have its data VGPRs overwritten by
a vector instruction right behind it.  A VMEM store reads its data registers
after it issues, and the ISA requires two wait states between a store of
more than 8 bytes and a vector write of those registers.  The compiler
inserts them after the stores it emits, but not after a store written in
inline asm (the device-scope non-temporal store), so that asm carries its
own s_nop; without it a schedule put a 64-bit VALU write (v_lshl_add_u64,
v_pk_mov_b32) on the next instruction and the store wrote the new values (an
FP4 dequantize variant stored its next address as data).

Compiles each kernel source to AMD assembly on the CPU (hipcc
cross-compiles) with the library's own flags."""
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
    subprocess.check_call([b.HIPCC, *b.FLAGS, *b.FILE_FLAGS.get(os.path.basename(src), []),
                           "-S", "--cuda-device-only", src, "-o", out],
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


_STORE = re.compile(r"^(?:global|buffer)_store_dword(?:x3|x4)\s+\S+\s+(v\[\d+:\d+\])")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _vector_dst(ins):
    parts = ins.replace(",", " ").split()
    if len(parts) < 2 or not parts[0].startswith("v_") or parts[0].startswith(("v_cmp", "v_readlane",
                                                                                 "v_readfirstlane")):
        return set()            # not a VALU op, or one whose result goes to SGPRs / VCC
    return _vregs(parts[1])


def _bodies(text):
    name, body = None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name, body = m.group(1), []
        elif name is not None and line.startswith(".Lfunc_end"):
            yield name, body
            name = None
        elif name is not None:
            code = line.split(";")[0].strip()
            if code and not code.startswith(".") and not code.endswith(":"):
                body.append(code)


def store_data_hazards(text, need=2):
    """(kernel, store, instruction) for every VALU write of a wide store's data
    VGPRs with fewer than `need` wait states between the two (`s_nop n` gives
    n + 1, any other instruction one)."""
    hits = []
    for name, body in _bodies(text):
        for i, ins in enumerate(body):
            m = _STORE.match(ins.replace(",", " "))
            if not m:
                continue
            data = _vregs(m.group(1))
            waited = 0
            for nxt in body[i + 1:]:
                if waited >= need:
                    break
                if nxt.startswith("s_nop"):
                    waited += int(nxt.split()[1], 0) + 1
                    continue
                if _vector_dst(nxt) & data:
                    hits.append((name, ins, nxt))
                    break
                waited += 1
    return hits


def test_store_hazard_detector():
    bad = ("_Z1kv:\n\tglobal_store_dwordx4 v[10:11], v[6:9], off nt sc1\n"
           "\tv_lshl_add_u64 v[6:7], v[0:1], 0, s[10:11]\n.Lfunc_end0:\n")
    assert len(store_data_hazards(bad)) == 1
    assert store_data_hazards(bad.replace("\tv_lshl", "\ts_nop 1\n\tv_lshl")) == []
    assert len(store_data_hazards(bad.replace("\tv_lshl", "\ts_nop 0\n\tv_lshl"))) == 1
    assert len(store_data_hazards(bad.replace("\tv_lshl", "\tv_mov_b32 v20, 0\n\tv_lshl"))) == 1
    assert store_data_hazards(bad.replace("\tv_lshl", "\tv_mov_b32 v20, 0\n\tv_mov_b32 v21, 0\n\tv_lshl")) == []
    assert store_data_hazards(bad.replace("v_lshl_add_u64 v[6:7]", "v_lshl_add_u64 v[12:13]")) == []
    assert store_data_hazards(bad.replace("dwordx4 v[10:11], v[6:9]", "dwordx2 v[10:11], v[6:7]")) == []


def test_no_store_data_hazard(listings):
    hits = [(os.path.basename(src),) + h for src, text in listings.items() for h in store_data_hazards(text)]
    assert not hits, "\n".join("%s %s\n    %s\n    %s" % h for h in hits[:10])
