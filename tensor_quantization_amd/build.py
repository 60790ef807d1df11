"""Build the gfx950 HIP library ``libtq.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled for gfx950 only, in parallel, then
linked into ``tensor_quantization_amd/libtq.so``.  Flags: -O3, no fast-math,
-ffp-contract=off (no a*b+c fusion: every binary32 step rounds as written),
and packed-fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wno-unused-command-line-argument",
]

# per-file extras: the GEMM keeps its matrix-core results in ordinary VGPRs,
# so the scale-and-accumulate step reads them without accumulator moves
FILE_FLAGS = {"tq_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, extra_flags=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every csrc/*.hip and link `out`; `extra_flags` (e.g. -D tunables)
    are appended to every compile line."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs, objs = [], []
    for s in srcs:
        o = os.path.join(build_dir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), *extra_flags, "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for s, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append(s)
            sys.stderr.write(text)
        elif verbose and lines:
            sys.stderr.write("\n".join(lines) + "\n")
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
