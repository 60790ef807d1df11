#!/usr/bin/env python3
"""Benchmark of the quantization hot path on one MI355X.

Headline (`value`): quantize GB/s of the per-token W8A8 workload -- bf16
[8192, 4096], N(0,1) with 1% outlier columns x20, symmetric s8 [-127, 127],
one fp32 scale per row.  A step is one quantize launch over the whole
tensor; `value` = algorithmic bytes (input read once + codes and scales
written once = 100,696,064 B) x K / wall time of K back-to-back launches
between two device synchronizations.  Inputs are resident in HBM before the
timed region and rotate over buffer sets (more than 1 GB in total, each set
re-read only after at least twice the 256 MB last-level cache of other
reads), so no launch is served from cache.

Also on the same JSON line:
  roofline       the quantize kernel: algorithmic bytes per launch / its mean
                 launch time from HIP events on the launch stream, against the
                 8 TB/s HBM peak; `traffic` = HBM bytes per launch from the
                 rocprofv3 counter summary in profiles/ (null when the
                 kernel's sources changed since).
  quantize       every workload's quantizer timed alone: per-tensor s8 f32
                 [64,256]; per-token s8; per-group u4 g=128 f16 [11008,4096];
                 FP8 1x128 bf16 [4096,7168] and 128x128 bf16 [7168,7168];
                 NVFP4 (static and dynamic per-tensor scale) and MXFP4 bf16
                 [14336,4096] -- each with its same-run streaming ceiling.
  copy_ceiling   the streaming ceiling kernel (tq_stream_mix) at each access
                 mix and size: what a plain stream with the kernel's per-lane
                 widths reaches on this chip in this run.
  path           the whole per-token path: quantize, dequantize to bf16, STE
                 backward (bf16 dy), dequantize backward, each kernel's GB/s.
  breakdown      every other op (dequantize, STE and dequantize backward of
                 each workload, transposes, FP4 follow-ons, fake quantization,
                 binary64, MXFP8, the consumer GEMMs), each timed alone on
                 inputs its producer wrote.
  cpu_baseline   the CPU oracle on a bounded row sample of each workload's
                 quantize, single-threaded and with its rows split over the
                 host's cores (OS threads, one oracle call per slice; the
                 oracle's arithmetic is unchanged), with the CPU model and the
                 SHA-256 of every input buffer.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-breakdown]
       [--no-cpu] [--only OP]
       python bench.py --trace-summary DIR     (rocprofv3 kernel-trace CSVs)
       python bench.py --pmc-summary DIR       (rocprofv3 counter CSVs)
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0      # dense fp8 (and int8) matrix-core peak
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 matrix-core peak
METRIC = "quantize GB/s (bytes in+out) & % HBM peak: per-token s8, g128 4-bit, FP4"
LLC_BYTES = 256 << 20
F32, F16, BF16 = 0, 1, 2
S8, U8, S4, U4 = 0, 1, 2, 3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None, help="time one op alone (profiling)")
    ap.add_argument("--iters", type=int, default=100, help="timed launches per op outside the headline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy 10 times (scales the HBM byte counters)")
    ap.add_argument("--trace-summary", default=None, help="summarize rocprofv3 kernel-trace CSVs under DIR")
    ap.add_argument("--pmc-summary", default=None, help="summarize rocprofv3 counter CSVs under DIR")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ helpers
def dev_bits(a, ft, torch):
    import numpy as np
    a = np.ascontiguousarray(a)
    if ft == "f32":
        return torch.from_numpy(a.copy()).cuda()
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[ft]
    return torch.from_numpy(a.view(np.int16).copy()).view(dt).cuda()


def P(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def nsets_for(read_bytes, set_bytes, cap_bytes=16 << 30):
    """Buffer sets to rotate so that a set's inputs are re-read only after at
    least twice the last-level cache of other reads (non-temporal stores do
    not allocate there, so reads alone must overflow it), and at least 1.2 GB
    in total; at most 64 sets (the tiny per-tensor workload is latency-bound
    and stays cache-resident) and cap_bytes of device memory."""
    n = max(4, 1 - (-2 * LLC_BYTES // max(1, read_bytes)), -(-int(1.2e9) // max(1, set_bytes)))
    return max(2, min(n, 64, cap_bytes // max(1, set_bytes)))


def replicate(base, n):
    """n buffer sets: `base` (inputs uploaded, producer outputs written) and
    n - 1 device copies of it."""
    return [base] + [{k: (v.clone() if hasattr(v, "clone") else v) for k, v in base.items()} for _ in range(n - 1)]


def set_bytes(s):
    return sum(v.numel() * v.element_size() for v in s.values() if hasattr(v, "numel"))


def check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed with status %d" % (what, rc))


def time_launches(torch, launch, sets, iters, warmup=20):
    """Mean launch time (us) of `iters` back-to-back launches rotating over
    `sets`, from one HIP event pair on the launch stream.  The untimed warmup
    launches touch every set once, so no timed launch is the first GPU access
    to its buffers (measured on the 66 MB FP4 transpose: 13.5 us per launch
    over 30 launches when most sets were first touched inside the timed
    region, 12.6 us over 200)."""
    n = len(sets)
    warmup = max(warmup, n)
    for i in range(warmup):
        launch(sets[i % n])
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a spin kernel ahead of the start event holds the stream while the host
    # enqueues every timed launch, so host-side call time cannot open gaps
    # between them; it ends before the start event and is not timed
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is not None:
        spin(min(40_000 * iters, 40_000_000))
    s_ev.record()
    for i in range(iters):
        launch(sets[(warmup + i) % n])
    e_ev.record()
    torch.cuda.synchronize()
    return 1000.0 * s_ev.elapsed_time(e_ev) / iters


def rate(nbytes, us):
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"bytes": nbytes, "us": round(us, 3), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


# Counter summaries in profiles/ hold a digest of the sources of the kernel
# they measured; a summary taken from other sources is stale.
KERNEL_SOURCES = {
    "quant_per_token_s8": ("tq_int.hip", "tq_device.h", "tq_host.h"),
    "quant_per_group_u4_g128": ("tq_int.hip", "tq_device.h", "tq_host.h"),
}


def source_digest(files=("tq_int.hip", "tq_device.h", "tq_host.h")):
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_quantization_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(op):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.txt" % op)
    if not os.path.exists(path) or op not in KERNEL_SOURCES:
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(KERNEL_SOURCES[op]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ inputs
class Inputs:
    """Every workload input, generated once on the host (seeded, see
    workloads/__init__.py) and kept for the GPU sets, the CPU samples and the
    SHA-256 record."""

    def __init__(self):
        self._a = {}

    def get(self, key):
        import numpy as np
        import workloads
        if key not in self._a:
            kind, name = key.split(":", 1)
            if kind == "x":
                self._a[key] = workloads.make_input(name)
            elif kind == "dy":
                self._a[key] = workloads.make_dy(name)
            elif kind == "f64":
                self._a[key] = np.random.default_rng(211).standard_normal((8192, 4096))
        return self._a[key]

    def sha256(self):
        return {k: hashlib.sha256(memoryview(v).cast("B")).hexdigest() for k, v in sorted(self._a.items())}


# ------------------------------------------------------------------ quantizers
def quantizers(torch, tq, inp):
    """(name, workload, algorithmic bytes, make base set, launch, reads,
    ceiling mix (in, out, store policy, threads)) for every workload's
    quantize call.  Inputs are generated when a set is first made."""
    import workloads
    L = tq._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    E = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")   # noqa: E731
    u8, f32 = torch.uint8, torch.float32
    shape = lambda key: tuple(workloads.CONFIGS[key]["shape"])           # noqa: E731
    ops = []

    R1, C1 = shape("c1_per_tensor_s8")
    n1 = R1 * C1
    ops.append(("per_tensor_s8", "f32 [64,256] per-tensor s8 (launch-bound)", n1 * 4 + n1 + 4,
                lambda: dict(x=dev_bits(inp.get("x:c1_per_tensor_s8"), "f32", torch), q=E(n1, u8), s=E(1, f32),
                             ws=E(8192, u8)),
                lambda b: check(L.tq_quant_per_tensor(P(b["x"]), F32, n1, S8, -127, 127, 0, P(b["q"]), P(b["s"]),
                                                      None, P(b["ws"]), 8192, stream), "c1 quant"),
                n1 * 4, None))

    R2, C2 = shape("c2_per_token_s8")
    n2 = R2 * C2
    ops.append(("per_token_s8", "bf16 [8192,4096] per-token s8", n2 * 3 + R2 * 4,
                lambda: dict(x=dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch), q=E((R2, C2), u8),
                             s=E(R2, f32)),
                lambda b: check(L.tq_quant_per_token(P(b["x"]), BF16, R2, C2, S8, -127, 127, P(b["q"]), P(b["s"]),
                                                     None, stream), "c2 quant"),
                n2 * 2, (16, 8, 1, n2 // 8)))

    N3, K3 = shape("c3_per_group_u4_g128")
    n3 = N3 * K3
    shp3 = (ctypes.c_int64 * 2)(N3, K3)
    ops.append(("per_group_u4_g128", "f16 [11008,4096] per-group u4 g=128 asymmetric", n3 * 2 + n3 // 2 +
                (n3 // 128) * 5,
                lambda: dict(x=dev_bits(inp.get("x:c3_per_group_u4_g128"), "f16", torch), q=E((N3, K3 // 2), u8),
                             s=E((N3, K3 // 128), f32), z=E((N3, K3 // 128), u8)),
                lambda b: check(L.tq_quant_per_group(P(b["x"]), F16, 2, shp3, 1, 128, U4, 0, 15, P(b["q"]), P(b["s"]),
                                                     P(b["z"]), stream), "c3 quant"),
                n3 * 2, (16, 4, 1, n3 // 8)))

    for key, name in (("c4_fp8_act_1x128", "fp8_1x128"), ("c4_fp8_weight_128x128", "fp8_128x128")):
        R, C = shape(key)
        br, bc = workloads.CONFIGS[key]["block"]
        ns = (R // br) * (C // bc)
        ops.append((name, "bf16 [%d,%d] FP8 E4M3 %dx%d" % (R, C, br, bc), R * C * 3 + ns * 4,
                    lambda key=key, R=R, C=C, ns=ns: dict(x=dev_bits(inp.get("x:" + key), "bf16", torch),
                                                          q=E((R, C), u8), s=E(ns, f32)),
                    lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_quant_fp8_block(P(b["x"]), BF16, R, C, br, bc,
                                                                                 P(b["q"]), P(b["s"]), stream),
                                                            "fp8 quant"),
                    R * C * 2, (16, 8, 1, R * C // 8)))

    N5, K5 = shape("c5_fp4_weight")
    n5 = N5 * K5
    for kind, gs in (("nvfp4", 16), ("mxfp4", 32)):
        nb = n5 * 2 + n5 // 2 + n5 // gs + (4 if kind == "nvfp4" else 0)
        mk = lambda gs=gs: dict(x=dev_bits(inp.get("x:c5_fp4_weight"), "bf16", torch),       # noqa: E731
                                p=E((N5, K5 // 2), u8), b=E((N5, K5 // gs), u8),
                                g=torch.full((1,), 1.2e-5, dtype=f32, device="cuda"), ws=E(8192, u8))
        cfg = "bf16 [14336,4096] %s" % kind.upper()
        if kind == "nvfp4":
            ops.append(("nvfp4_static_global", cfg + " (static per-tensor scale)", nb, mk,
                        lambda b: check(L.tq_quant_fp4_block(P(b["x"]), BF16, N5, K5, 0, P(b["p"]), P(b["b"]), P(b["g"]),
                                                             1, None, 0, stream), "nvfp4 static"),
                        n5 * 2, (16, 4, 1, n5 // 8)))
            ops.append(("nvfp4_dynamic_global", cfg + " (per-tensor scale from the data: max pass + encode)", nb, mk,
                        lambda b: check(L.tq_quant_fp4_block(P(b["x"]), BF16, N5, K5, 0, P(b["p"]), P(b["b"]), P(b["g"]),
                                                             0, P(b["ws"]), 8192, stream), "nvfp4 dynamic"),
                        n5 * 2, (16, 4, 1, n5 // 8)))
        else:
            ops.append(("mxfp4", cfg, nb, mk,
                        lambda b: check(L.tq_quant_fp4_block(P(b["x"]), BF16, N5, K5, 1, P(b["p"]), P(b["b"]), None, 1,
                                                             None, 0, stream), "mxfp4"),
                        n5 * 2, (16, 4, 1, n5 // 8)))
    return ops


def run_quantizers(torch, tq, inp, steps, warmup, iters, only=None):
    """The headline per-token quantize over exactly `steps` launches after
    `warmup`, then every quantizer and its same-size streaming ceiling."""
    ops = quantizers(torch, tq, inp)
    out, head = {}, None
    ceil_cache = {}
    for name, cfg, nbytes, mk, launch, reads, mix in ops:
        if only and only != "quant_" + name:
            continue
        log("quantize:", name)
        base = mk()
        sets = replicate(base, nsets_for(reads, set_bytes(base)))
        if name == "per_token_s8":
            n = len(sets)
            for i in range(warmup):
                launch(sets[i % n])
            s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            s_ev.record()
            for i in range(steps):
                launch(sets[(warmup + i) % n])
            e_ev.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            us = 1000.0 * s_ev.elapsed_time(e_ev) / steps
            head = (nbytes, wall, us)
        else:
            us = time_launches(torch, launch, sets, iters)
        d = rate(nbytes, us)
        d["workload"] = cfg
        del sets, base
        torch.cuda.empty_cache()
        if mix is not None and not only:
            if mix not in ceil_cache:
                ceil_cache[mix] = stream_ceiling(torch, tq, *mix, iters=iters)
            c = ceil_cache[mix]
            d["ceiling"] = {"mix": "%d:%d per unit" % mix[:2], "GBps": c["GBps"], "frac": c["frac"],
                            "units_per_lane": c["units_per_lane"], "store_policy": c["store_policy"]}
            d["of_ceiling"] = round(d["GBps"] / c["GBps"], 4)
        t = read_traffic("quant_" + name)
        if t is not None:
            d["traffic"] = t
        out[name] = d
    return out, head, ceil_cache


# ------------------------------------------------------------------ ceilings
def stream_ceiling(torch, tq, in_b, out_b, policy, nthr, iters=100):
    """The streaming ceiling of one access mix at one size: the best of the
    stream kernel with 1, 2 and 4 units per lane and, for 16-byte stores, both
    non-temporal store policies (each shape's figure kept)."""
    L = tq._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    src_bytes = nthr * in_b
    base = dict(src=torch.empty(src_bytes, dtype=torch.uint8, device="cuda"),
                dst=torch.empty(nthr * out_b, dtype=torch.uint8, device="cuda"))
    base["src"].fill_(0x3c)
    sets = replicate(base, nsets_for(src_bytes, set_bytes(base)))
    policies = [policy] + ([3 - policy] if out_b >= 16 and policy in (1, 2) else [])
    shapes = {}
    for pol in policies:
        for v in (1, 2, 4):
            us = time_launches(torch, lambda b, v=v, pol=pol: check(L.tq_stream_mix(
                P(b["src"]), P(b["dst"]), nthr, in_b, out_b, pol, v, stream), "stream mix"), sets, iters)
            shapes[(pol, v)] = rate(nthr * (in_b + out_b), us)
    del sets, base
    torch.cuda.empty_cache()
    best = min(shapes, key=lambda k: shapes[k]["us"])
    d = dict(shapes[best])
    d["mix"] = "%d:%d bytes per unit, %d units" % (in_b, out_b, nthr)
    d["store_policy"], d["units_per_lane"] = best
    d["GBps_by_shape"] = {"policy%d_x%d" % k: shapes[k]["GBps"] for k in shapes}
    return d


CEILINGS = [
    # name, in, out, store policy, lanes
    ("quantize_8bit_per_token", 16, 8, 1, 8192 * 4096 // 8),
    ("quantize_4bit_g128", 16, 4, 1, 11008 * 4096 // 8),
    ("quantize_4bit_fp4", 16, 4, 1, 14336 * 4096 // 8),
    ("dequantize_8bit_per_token", 8, 16, 2, 8192 * 4096 // 8),
    ("dequantize_4bit_g128", 4, 16, 1, 11008 * 4096 // 8),
    ("dequantize_4bit_fp4", 4, 16, 1, 14336 * 4096 // 8),
    ("ste_backward_per_token", 32, 16, 1, 8192 * 4096 // 8),
    ("dequantize_backward_per_token", 16, 16, 2, 8192 * 4096 // 8),
    ("copy_1to1_fp4_transpose_size", 16, 16, 1, 2 * (14336 * 2048 + 14336 * 256) // 32),
]


# ------------------------------------------------------------------ per-token path
def build_path(torch, tq, inp):
    x = inp.get("x:c2_per_token_s8")
    dy = inp.get("dy:c2_per_token_s8")
    rows, cols = x.shape
    L = tq._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    base = dict(x=dev_bits(x, "bf16", torch), dy=dev_bits(dy, "bf16", torch),
                q=torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
                s=torch.empty(rows, dtype=torch.float32, device="cuda"),
                y=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
                dx=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
                dq=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"))
    n = rows * cols
    kernels = {
        "quant_per_token_s8": (n * 2 + n + rows * 4, lambda b: check(L.tq_quant_per_token(
            P(b["x"]), BF16, rows, cols, S8, -127, 127, P(b["q"]), P(b["s"]), None, stream), "quant")),
        "dequant_per_token_s8": (n + rows * 4 + n * 2, lambda b: check(L.tq_dequant_per_token(
            P(b["q"]), S8, rows, cols, P(b["s"]), None, P(b["y"]), BF16, stream), "dequant")),
        "quant_per_token_s8_backward": (n * 2 * 3 + rows * 4, lambda b: check(L.tq_quant_per_token_backward(
            P(b["x"]), BF16, rows, cols, S8, -127, 127, P(b["s"]), None, P(b["dy"]), P(b["dx"]), stream), "ste")),
        "dequant_per_token_backward": (n * 2 * 2 + rows * 4, lambda b: check(L.tq_dequant_per_token_backward(
            P(b["dy"]), BF16, rows, cols, P(b["s"]), P(b["dq"]), stream), "dqb")),
    }
    kernels["quant_per_token_s8"][1](base)          # the codes and scales the consumers read
    torch.cuda.synchronize()
    sets = replicate(base, nsets_for(n, set_bytes(base)))   # smallest read stream: the s8 codes
    return sets, kernels


def run_path(torch, tq, inp, steps):
    """The four kernels of the per-token path, K launches each, issued kernel
    by kernel (K quantize, K dequantize, ...): the same work and dependency
    order as K whole passes.  One launch counter picks the buffer set, so
    every launch reads the set touched longest ago."""
    sets, kernels = build_path(torch, tq, inp)
    names = list(kernels)
    c = 0
    for _ in range(3):
        for k in names:
            kernels[k][1](sets[c % len(sets)])
            c += 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for j, k in enumerate(names):
        for _ in range(steps):
            kernels[k][1](sets[c % len(sets)])
            c += 1
        ev[j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = {k: rate(kernels[k][0], 1000.0 * ev[j].elapsed_time(ev[j + 1]) / steps) for j, k in enumerate(names)}
    path_bytes = sum(kernels[k][0] for k in names)
    del sets
    torch.cuda.empty_cache()
    return {"workload": "bf16 [8192,4096] per-token s8: quantize + dequantize(bf16) + STE backward(bf16 dy) + "
                        "dequantize backward", "bytes_per_pass": path_bytes, "passes": steps,
            "GBps": round(path_bytes * steps / wall / 1e9, 1), "frac": round(path_bytes * steps / wall / 1e9 /
                                                                            HBM_PEAK_GBPS, 4),
            "kernels": per_kernel}


# ------------------------------------------------------------------ breakdown
def breakdown(torch, tq, inp, iters=100, only=None, ceil_cache=None):
    """Every other op timed alone; each buffer set holds what the op's
    producer (the matching quantize call) wrote.  A streaming op with a
    `mix` (bytes read and written per unit, store policy, units at its size)
    also gets the same-run streaming ceiling of that mix (`ceiling`,
    `of_ceiling`); `ceil_cache` shares ceilings already measured."""
    import numpy as np
    L = tq._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []

    ceil_cache = {} if ceil_cache is None else ceil_cache

    def bench_op(name, cfg, nbytes, make_base, launch, read_bytes, flops=None, peak=FP8_PEAK_TFLOPS, mix=None):
        if only and only != name:
            return
        log("breakdown:", name)
        base = make_base()
        torch.cuda.synchronize()
        sets = replicate(base, nsets_for(read_bytes, set_bytes(base)))
        us = time_launches(torch, launch, sets, iters)
        if flops is None:
            d = dict(op=name, workload=cfg, **rate(nbytes, us))
            del sets, base
            torch.cuda.empty_cache()
            if mix is not None and not only:
                if mix not in ceil_cache:
                    ceil_cache[mix] = stream_ceiling(torch, tq, *mix, iters=iters)
                c = ceil_cache[mix]
                d["ceiling"] = {"mix": "%d:%d per unit, %d units" % (mix[0], mix[1], mix[3]), "GBps": c["GBps"],
                                "frac": c["frac"], "units_per_lane": c["units_per_lane"],
                                "store_policy": c["store_policy"]}
                d["of_ceiling"] = round(d["GBps"] / c["GBps"], 4)
            out.append(d)
            return
        tf = flops / (us * 1e-6) / 1e12
        out.append({"op": name, "workload": cfg, "flops": flops, "us": round(us, 3), "TFLOPs": round(tf, 1),
                    "frac": round(tf / peak, 4), "bound": "mfma"})
        del sets, base
        torch.cuda.empty_cache()

    E = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")   # noqa: E731
    u8, f32, bf16, f16 = torch.uint8, torch.float32, torch.bfloat16, torch.float16

    # per-tensor s8, f32 [64, 256]: STE, dequantize, dequantize backward on
    # the quantizer's scale and codes
    import workloads
    shape = lambda key: tuple(workloads.CONFIGS[key]["shape"])           # noqa: E731
    n1 = int(np.prod(shape("c1_per_tensor_s8")))

    def mk1():
        b = dict(x=dev_bits(inp.get("x:c1_per_tensor_s8"), "f32", torch),
                 dy=dev_bits(inp.get("dy:c1_per_tensor_s8"), "f32", torch), q=E(n1, u8), s=E(1, f32),
                 ws=E(8192, u8), y=E(n1, f32), dx=E(n1, f32))
        check(L.tq_quant_per_tensor(P(b["x"]), F32, n1, S8, -127, 127, 0, P(b["q"]), P(b["s"]), None, P(b["ws"]),
                                    8192, stream), "c1 producer")
        return b
    cfg1 = "f32 [64,256] per-tensor s8"
    bench_op("quant_per_tensor_s8_backward", cfg1, n1 * 12 + 4, mk1,
             lambda b: check(L.tq_quant_per_tensor_backward(P(b["x"]), F32, n1, S8, -127, 127, P(b["s"]), None,
                                                            P(b["dy"]), P(b["dx"]), stream), "c1 ste"), n1 * 8)
    bench_op("dequant_per_tensor_s8", cfg1, n1 * 5 + 4, mk1,
             lambda b: check(L.tq_dequant_per_tensor(P(b["q"]), S8, n1, P(b["s"]), None, P(b["y"]), F32, stream),
                             "c1 deq"), n1)

    # per-token s8 on bf16 [8192, 4096]: fake quantization (round trip) and
    # its backward at per-tensor scope
    n2 = int(np.prod(shape("c2_per_token_s8")))

    def mkf2():
        b = dict(x=dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch),
                 dy=dev_bits(inp.get("dy:c2_per_token_s8"), "bf16", torch), y=E(n2, bf16), s=E(1, f32),
                 ws=E(8192, u8), dx=E(n2, bf16))
        check(L.tq_fake_quant_per_tensor(P(b["x"]), BF16, n2, S8, -127, 127, 0, P(b["y"]), P(b["s"]), None,
                                         P(b["ws"]), 8192, stream), "fake producer")
        return b
    cfg2 = "bf16 [8192,4096] per-tensor s8"
    bench_op("fake_quant_per_tensor_s8_dynamic", cfg2, n2 * 4 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor(P(b["x"]), BF16, n2, S8, -127, 127, 0, P(b["y"]), P(b["s"]),
                                                        None, P(b["ws"]), 8192, stream), "fake dyn"), n2 * 2)
    bench_op("fake_quant_per_tensor_s8_static", cfg2, n2 * 4 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor(P(b["x"]), BF16, n2, S8, -127, 127, 1, P(b["y"]), P(b["s"]),
                                                        None, None, 0, stream), "fake static"), n2 * 2,
             mix=(16, 16, 1, n2 // 8))
    bench_op("fake_quant_per_tensor_s8_backward", cfg2, n2 * 6 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor_backward(P(b["x"]), BF16, n2, S8, -127, 127, P(b["s"]), None,
                                                                 P(b["dy"]), P(b["dx"]), stream), "fake bwd"),
             n2 * 4, mix=(32, 16, 1, n2 // 8))

    # per-tensor FP8 E4M3 on the same bf16 [8192, 4096] input: the dynamic
    # scale (chunk maxima, then the encode merging them) and a static one
    def mkq8t():
        b = dict(x=dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch), q=E(n2, u8), s=E(1, f32),
                 ws=E(8192, u8))
        check(L.tq_quant_fp8_per_tensor(P(b["x"]), BF16, n2, 0, P(b["q"]), P(b["s"]), P(b["ws"]), 8192, stream),
              "fp8 per-tensor producer")
        return b
    cfg8 = "bf16 [8192,4096] per-tensor FP8 E4M3"
    bench_op("quant_fp8_per_tensor_dynamic", cfg8, n2 * 3 + 4, mkq8t,
             lambda b: check(L.tq_quant_fp8_per_tensor(P(b["x"]), BF16, n2, 0, P(b["q"]), P(b["s"]), P(b["ws"]), 8192,
                                                       stream), "fp8 per-tensor dyn"), n2 * 2)
    bench_op("quant_fp8_per_tensor_static", cfg8, n2 * 3 + 4, mkq8t,
             lambda b: check(L.tq_quant_fp8_per_tensor(P(b["x"]), BF16, n2, 1, P(b["q"]), P(b["s"]), None, 0,
                                                       stream), "fp8 per-tensor static"), n2 * 2,
             mix=(16, 8, 1, n2 // 8))

    # binary64 inputs: the per-token workload's shape in f64 (N(0,1) values)
    shpf = (ctypes.c_int64 * 2)(8192, 4096)

    def mkd():
        b = dict(x=torch.from_numpy(inp.get("f64:per_token")).cuda(), q=E(n2, u8), s=E(8192, torch.float64), y=E((8192, 4096), torch.float64))
        check(L.tq_quant_f64(P(b["x"]), 2, shpf, 2, 0, 0, S8, -127, 127, 0, P(b["q"]), P(b["s"]), None, None, 0,
                             stream), "f64 producer")
        return b
    cfgf = "f64 [8192,4096] per-token s8"
    bench_op("quant_f64_per_token_s8", cfgf, n2 * 9 + 8192 * 8, mkd,
             lambda b: check(L.tq_quant_f64(P(b["x"]), 2, shpf, 2, 0, 0, S8, -127, 127, 0, P(b["q"]), P(b["s"]), None,
                                            None, 0, stream), "f64 quant"), n2 * 8)
    bench_op("dequant_f64_per_token_s8", cfgf, n2 * 9 + 8192 * 8, mkd,
             lambda b: check(L.tq_dequant_f64(P(b["q"]), S8, 2, shpf, 2, 0, 0, P(b["s"]), None, P(b["y"]), stream),
                             "f64 dequant"), n2)

    # per-group u4 g128 asymmetric, f16 [11008, 4096]: dequantize to f16
    N3, K3 = shape("c3_per_group_u4_g128")
    n3 = N3 * K3
    shp3 = (ctypes.c_int64 * 2)(N3, K3)
    b3 = n3 * 2 + n3 // 2 + (n3 // 128) * 5

    def mk3():
        b = dict(x=dev_bits(inp.get("x:c3_per_group_u4_g128"), "f16", torch), q=E((N3, K3 // 2), u8),
                 s=E((N3, K3 // 128), f32),
                 z=E((N3, K3 // 128), u8), y=E((N3, K3), f16))
        check(L.tq_quant_per_group(P(b["x"]), F16, 2, shp3, 1, 128, U4, 0, 15, P(b["q"]), P(b["s"]), P(b["z"]),
                                   stream), "c3 producer")
        del b["x"]
        return b
    bench_op("dequant_per_group_u4_g128", "f16 [11008,4096] per-group u4 g=128", b3, mk3,
             lambda b: check(L.tq_dequant_per_group(P(b["q"]), U4, 2, shp3, 1, 128, P(b["s"]), P(b["z"]), P(b["y"]),
                                                    F16, stream), "c3 dequant"), n3 // 2 + (n3 // 128) * 5,
             mix=(4, 16, 1, n3 // 8))

    # and its two backward rules on the same codes: STE (f16 x, dy -> dx) and
    # dequantize backward (f16 dy -> dq)
    def mk3x():
        b = dict(x=dev_bits(inp.get("x:c3_per_group_u4_g128"), "f16", torch),
                 dy=dev_bits(inp.get("dy:c3_per_group_u4_g128"), "f16", torch), q=E((N3, K3 // 2), u8),
                 s=E((N3, K3 // 128), f32), z=E((N3, K3 // 128), u8), dx=E((N3, K3), f16))
        check(L.tq_quant_per_group(P(b["x"]), F16, 2, shp3, 1, 128, U4, 0, 15, P(b["q"]), P(b["s"]), P(b["z"]),
                                   stream), "c3 producer")
        del b["q"]
        return b
    cfg3 = "f16 [11008,4096] per-group u4 g=128"
    bench_op("quant_backward_per_group_u4_g128", cfg3, n3 * 6 + (n3 // 128) * 5, mk3x,
             lambda b: check(L.tq_quant_per_group_backward(P(b["x"]), F16, 2, shp3, 1, 128, U4, 0, 15, P(b["s"]),
                                                           P(b["z"]), P(b["dy"]), P(b["dx"]), stream), "c3 ste"),
             n3 * 4 + (n3 // 128) * 5, mix=(32, 16, 1, n3 // 8))
    bench_op("dequant_backward_per_group_g128", cfg3, n3 * 4 + (n3 // 128) * 4, mk3x,
             lambda b: check(L.tq_dequant_per_group_backward(P(b["dy"]), F16, 2, shp3, 1, 128, P(b["s"]), P(b["dx"]),
                                                             stream), "c3 dqb"),
             n3 * 2 + (n3 // 128) * 4, mix=(16, 16, 2, n3 // 8))

    # FP8 1x128 activations bf16 [4096, 7168]; 128x128 weights bf16 [7168, 7168]
    for key, name in (("c4_fp8_act_1x128", "fp8_1x128"), ("c4_fp8_weight_128x128", "fp8_128x128")):
        R, C = shape(key)
        br, bc = workloads.CONFIGS[key]["block"]
        ns = (R // br) * (C // bc)
        nb = R * C * 3 + ns * 4

        def mk(key=key, R=R, C=C, ns=ns, br=br, bc=bc):
            b = dict(x=dev_bits(inp.get("x:" + key), "bf16", torch), dy=dev_bits(inp.get("dy:" + key), "bf16", torch),
                     q=E((R, C), u8), s=E(ns, f32),
                     y=E((R, C), bf16))
            check(L.tq_quant_fp8_block(P(b["x"]), BF16, R, C, br, bc, P(b["q"]), P(b["s"]), stream), "fp8 producer")
            return b
        cfg = "bf16 [%d,%d] FP8 %dx%d" % (R, C, br, bc)
        bench_op("dequant_" + name, cfg, nb, mk,
                 lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_dequant_fp8_block(P(b["q"]), R, C, br, bc, P(b["s"]),
                                                                                P(b["y"]), BF16, stream), "fp8 deq"),
                 R * C + ns * 4, mix=(8, 16, 2, R * C // 8))
        if name == "fp8_1x128":
            bench_op("quant_backward_" + name, cfg, R * C * 6 + ns * 4, mk,
                     lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_quant_fp8_block_backward(
                         P(b["x"]), BF16, R, C, br, bc, P(b["s"]), P(b["dy"]), P(b["y"]), stream), "fp8 ste"),
                     R * C * 4 + ns * 4, mix=(32, 16, 1, R * C // 8))
            bench_op("dequant_backward_" + name, cfg, R * C * 4 + ns * 4, mk,
                     lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_dequant_fp8_block_backward(
                         P(b["dy"]), BF16, R, C, br, bc, P(b["s"]), P(b["y"]), stream), "fp8 dqb"),
                     R * C * 2 + ns * 4, mix=(16, 16, 2, R * C // 8))

    # MXFP8 on the FP8 activation workload bf16 [4096, 7168]: E4M3 + E8M0 per 32
    Rm, Cm = shape("c4_fp8_act_1x128")
    nm = Rm * Cm
    bm = nm * 2 + nm + nm // 32

    def mkm():
        b = dict(x=dev_bits(inp.get("x:c4_fp8_act_1x128"), "bf16", torch), q=E((Rm, Cm), u8), b=E((Rm, Cm // 32), u8),
                 y=E((Rm, Cm), bf16))
        check(L.tq_quant_mxfp8(P(b["x"]), BF16, Rm, Cm, P(b["q"]), P(b["b"]), stream), "mxfp8 producer")
        return b
    bench_op("quant_mxfp8", "bf16 [4096,7168] MXFP8", bm, mkm,
             lambda b: check(L.tq_quant_mxfp8(P(b["x"]), BF16, Rm, Cm, P(b["q"]), P(b["b"]), stream), "mxfp8"),
             nm * 2, mix=(16, 8, 1, nm // 8))
    bench_op("dequant_mxfp8", "bf16 [4096,7168] MXFP8", bm, mkm,
             lambda b: check(L.tq_dequant_mxfp8(P(b["q"]), P(b["b"]), Rm, Cm, P(b["y"]), BF16, stream), "mxfp8 deq"),
             nm + nm // 32, mix=(8, 16, 1, nm // 8))

    def mkm2():
        b = mkm()
        b["dy"] = dev_bits(inp.get("dy:c4_fp8_act_1x128"), "bf16", torch)
        return b
    bench_op("quant_backward_mxfp8", "bf16 [4096,7168] MXFP8", nm * 6 + nm // 32, mkm2,
             lambda b: check(L.tq_quant_mxfp8_backward(P(b["x"]), BF16, P(b["b"]), Rm, Cm, P(b["dy"]), P(b["y"]),
                                                       stream), "mxfp8 ste"),
             nm * 4 + nm // 32, mix=(32, 16, 1, nm // 8))
    bench_op("dequant_backward_mxfp8", "bf16 [4096,7168] MXFP8", nm * 4 + nm // 32, mkm2,
             lambda b: check(L.tq_dequant_mxfp8_backward(P(b["dy"]), BF16, P(b["b"]), Rm, Cm, P(b["y"]), stream),
                             "mxfp8 dqb"),
             nm * 2 + nm // 32, mix=(16, 16, 2, nm // 8))

    # FP4 weight bf16 [14336, 4096]: dequantize, STE, dequantize backward and
    # the GEMM-layout transposes on the quantizer's outputs
    N5, K5 = shape("c5_fp4_weight")
    n5 = N5 * K5
    for kind, gs in (("nvfp4", 16), ("mxfp4", 32)):
        kd = 0 if kind == "nvfp4" else 1

        def mk(gs=gs, kd=kd, with_x=False):
            b = dict(x=dev_bits(inp.get("x:c5_fp4_weight"), "bf16", torch), p=E((N5, K5 // 2), u8),
                     b=E((N5, K5 // gs), u8), g=E(1, f32), ws=E(8192, u8), pt=E((K5 // 2, N5), u8), bt=E((K5 // gs, N5), u8),
                     y=E((N5, K5), bf16))
            check(L.tq_quant_fp4_block(P(b["x"]), BF16, N5, K5, kd, P(b["p"]), P(b["b"]), P(b["g"]), 0, P(b["ws"]),
                                       8192, stream), "fp4 producer")
            if with_x:
                b["dy"] = dev_bits(inp.get("dy:c5_fp4_weight"), "bf16", torch)
            else:
                del b["x"]
            return b
        cfg = "bf16 [14336,4096] %s" % kind.upper()
        gp = (lambda b: P(b["g"])) if kind == "nvfp4" else (lambda b: None)
        db = n5 // 2 + n5 // gs + (4 if kind == "nvfp4" else 0) + n5 * 2
        bench_op("dequant_" + kind, cfg, db, mk,
                 lambda b, kd=kd, gp=gp: check(L.tq_dequant_fp4_block(P(b["p"]), P(b["b"]), gp(b), N5, K5, kd,
                                                                      P(b["y"]), BF16, stream), "fp4 dequant"),
                 n5 // 2 + n5 // gs, mix=(4, 16, 1, n5 // 8))
        mkx = lambda mk=mk: mk(with_x=True)   # noqa: E731
        gb4 = 4 if kind == "nvfp4" else 0
        bench_op("quant_backward_" + kind, cfg, n5 * 6 + n5 // gs + gb4, mkx,
                 lambda b, kd=kd, gp=gp: check(L.tq_quant_fp4_block_backward(P(b["x"]), BF16, P(b["b"]), gp(b), N5, K5,
                                                                             kd, P(b["dy"]), P(b["y"]), stream),
                                               "fp4 ste"),
                 n5 * 4 + n5 // gs, mix=(32, 16, 1, n5 // 8))
        bench_op("dequant_backward_" + kind, cfg, n5 * 4 + n5 // gs + gb4, mkx,
                 lambda b, kd=kd, gp=gp: check(L.tq_dequant_fp4_block_backward(P(b["dy"]), BF16, P(b["b"]), gp(b), N5,
                                                                               K5, kd, P(b["y"]), stream), "fp4 dqb"),
                 n5 * 2 + n5 // gs, mix=(16, 16, 2, n5 // 8))
        tb = 2 * (n5 // 2 + n5 // gs)
        bench_op("transpose_for_gemm_" + kind, cfg, tb, mk,
                 lambda b, gs=gs: check(L.tq_fp4_transpose_for_gemm(P(b["p"]), P(b["b"]), N5, K5, gs, P(b["pt"]),
                                                                    P(b["bt"]), stream), "transpose"),
                 tb // 2, mix=(16, 16, 1, tb // 32))

    # FP4 layout follow-ons on the NVFP4 weight: two weights (the quantized
    # weight and its row reversal) fused into one [2048, 28672] GEMM operand,
    # stacked by rows, and the FP8 expansion
    pb, sbb = n5 // 2, n5 // 16
    sg5 = {}

    def mkf():
        b = dict(x=dev_bits(inp.get("x:c5_fp4_weight"), "bf16", torch), p1=E((N5, K5 // 2), u8),
                 b1=E((N5, K5 // 16), u8), g=E(1, f32),
                 ws=E(8192, u8))
        check(L.tq_quant_fp4_block(P(b["x"]), BF16, N5, K5, 0, P(b["p1"]), P(b["b1"]), P(b["g"]), 0, P(b["ws"]),
                                   8192, stream), "nvfp4 producer")
        del b["x"], b["ws"]
        b["p2"], b["b2"] = torch.flip(b["p1"], [0]).contiguous(), torch.flip(b["b1"], [0]).contiguous()
        b.update(pt=E((K5 // 2, 2 * N5), u8), bt=E((K5 // 16, 2 * N5), u8), po=E((2 * N5, K5 // 2), u8),
                 bo=E((2 * N5, K5 // 16), u8), f8=E((N5, K5), u8))
        torch.cuda.synchronize()
        sg5["g"] = float(b["g"].item())
        return b
    cfgf = "NVFP4 2 x [14336,4096]"

    def concat_t(b):
        pp = (ctypes.c_void_p * 2)(b["p1"].data_ptr(), b["p2"].data_ptr())
        bb = (ctypes.c_void_p * 2)(b["b1"].data_ptr(), b["b2"].data_ptr())
        nn = (ctypes.c_int64 * 2)(N5, N5)
        check(L.tq_fp4_transpose_concat_for_gemm(2, pp, bb, nn, K5, 16, 128, P(b["pt"]), P(b["bt"]), None,
                                                 stream), "transpose concat")
    bench_op("transpose_concat_for_gemm_nvfp4", cfgf, 4 * (pb + sbb), mkf, concat_t, 2 * (pb + sbb),
             mix=(16, 16, 1, 4 * (pb + sbb) // 32))
    bench_op("concat_rows_nvfp4", cfgf, 4 * (pb + sbb), mkf,
             lambda b: check(L.tq_fp4_concat_rows(P(b["p1"]), P(b["b1"]), sg5["g"], P(b["p2"]), P(b["b2"]), sg5["g"],
                                                  N5, N5, K5, P(b["po"]), P(b["bo"]), stream), "concat rows"),
             2 * (pb + sbb), mix=(16, 16, 1, 4 * (pb + sbb) // 32))
    bench_op("predequant_to_fp8_nvfp4", "NVFP4 [14336,4096]", pb + sbb + n5, mkf,
             lambda b: check(L.tq_fp4_predequant_to_fp8(P(b["p1"]), P(b["b1"]), sg5["g"], N5, K5, 0, P(b["f8"]),
                                                        stream), "predequant"),
             pb + sbb)

    # block-scaled FP8 GEMM: the FP8 activations [4096, 7168] (1 x 128) times
    # the FP8 weight [7168, 7168] (128 x 128), bf16 out; 2 M N K flops
    if not only or only == "fp8_block_gemm":
        Mg, Kg = 4096, 7168
        Ng = Kg

        def mkg():
            xa = dev_bits(inp.get("x:c4_fp8_act_1x128"), "bf16", torch)
            xw = dev_bits(inp.get("x:c4_fp8_weight_128x128"), "bf16", torch)
            qa, sa = tq.tq_quant_fp8_block(xa, 1, 128)
            qw, sw = tq.tq_quant_fp8_block(xw, 128, 128)
            return dict(qa=qa, sa=sa, qw=qw, sw=sw, y=E((Mg, Ng), bf16))
        gb = Mg * Kg + Ng * Kg + 2 * Mg * Ng + 4 * (Mg * Kg // 128 + Ng * Kg // 16384)
        bench_op("fp8_block_gemm", "fp8 [4096,7168] x [7168,7168]^T bf16 out", gb, mkg,
                 lambda b: check(L.tq_fp8_block_gemm(P(b["qa"]), P(b["sa"]), P(b["qw"]), P(b["sw"]), Mg, Ng, Kg,
                                                     P(b["y"]), BF16, stream), "fp8 gemm"),
                 Mg * Kg + Ng * Kg, flops=2 * Mg * Ng * Kg)

    # W8A8 quantized linear: the per-token s8 activations [8192, 4096] times
    # the per-group weight's f16 values [11008, 4096] quantized per channel
    # to s8, bf16 out
    if not only or only == "w8a8_linear":
        Mq, Kq, Nq = 8192, 4096, 11008

        def mkq():
            qx, sx, _ = tq.tq_quant_per_token(dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch))
            qw, sw, _ = tq.tq_quant_per_token(dev_bits(inp.get("x:c3_per_group_u4_g128"), "f16", torch))
            return dict(qx=qx, sx=sx, qw=qw, sw=sw, y=E((Mq, Nq), bf16))
        qb = Mq * Kq + Nq * Kq + 2 * Mq * Nq + 4 * (Mq + Nq)
        bench_op("w8a8_linear", "s8 [8192,4096] x s8 [11008,4096]^T bf16 out", qb, mkq,
                 lambda b: check(L.tq_w8a8_linear(P(b["qx"]), P(b["sx"]), P(b["qw"]), P(b["sw"]), Mq, Nq, Kq,
                                                  P(b["y"]), BF16, stream), "w8a8"),
                 Mq * Kq + Nq * Kq, flops=2 * Mq * Nq * Kq)

    # FP4 weight-only linear: bf16 activations [8192, 4096] (the per-token
    # workload) times the NVFP4 weight [14336, 4096], bf16 out
    if not only or only == "fp4_linear_nvfp4":
        Mf, Kf, Nf = 8192, 4096, 14336

        def mkf4():
            xf0 = dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch)
            p, b_, g = tq.tq_quant_fp4_block(dev_bits(inp.get("x:c5_fp4_weight"), "bf16", torch), "nvfp4")
            return dict(x=xf0, p=p, b=b_, g=g, y=E((Mf, Nf), bf16))
        fb4 = Mf * Kf * 2 + Nf * Kf // 2 + Nf * Kf // 16 + 2 * Mf * Nf
        bench_op("fp4_linear_nvfp4", "bf16 [8192,4096] x nvfp4 [14336,4096]^T bf16 out", fb4, mkf4,
                 lambda b: check(L.tq_fp4_linear(P(b["x"]), BF16, P(b["p"]), P(b["b"]), P(b["g"]), 0, Mf, Nf, Kf,
                                                 P(b["y"]), BF16, stream), "fp4 linear"),
                 Mf * Kf * 2 + Nf * Kf // 2, flops=2 * Mf * Nf * Kf, peak=BF16_PEAK_TFLOPS)
    if not only or only == "fp4_linear_mxfp4":
        Mf, Kf, Nf = 8192, 4096, 14336

        def mkm4():
            xf0 = dev_bits(inp.get("x:c2_per_token_s8"), "bf16", torch)
            p, b_, _ = tq.tq_quant_fp4_block(dev_bits(inp.get("x:c5_fp4_weight"), "bf16", torch), "mxfp4")
            return dict(x=xf0, p=p, b=b_, y=E((Mf, Nf), bf16))
        fm4 = Mf * Kf * 2 + Nf * Kf // 2 + Nf * Kf // 32 + 2 * Mf * Nf
        bench_op("fp4_linear_mxfp4", "bf16 [8192,4096] x mxfp4 [14336,4096]^T bf16 out", fm4, mkm4,
                 lambda b: check(L.tq_fp4_linear(P(b["x"]), BF16, P(b["p"]), P(b["b"]), None, 1, Mf, Nf, Kf,
                                                 P(b["y"]), BF16, stream), "fp4 linear mx"),
                 Mf * Kf * 2 + Nf * Kf // 2, flops=2 * Mf * Nf * Kf, peak=BF16_PEAK_TFLOPS)
    return out


# ------------------------------------------------------------------ CPU
def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, os.cpu_count(), avail


def cpu_baseline(inp):
    """The oracle's quantize on a bounded leading-row sample of each
    workload: best of 3 wall times single-threaded, then with the sample's
    rows (whole groups / tiles) split over the host's threads, one oracle call
    per slice (ctypes releases the interpreter lock, so the slices run at
    once).  GB/s over the same algorithmic bytes as the GPU figures."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    oracle.lib()
    model, ncpu, avail = cpu_info()
    nthr = max(1, min(avail, 16))

    def best(fn, reps=3):
        t = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
        return min(t)

    def split(rows, unit):
        """Row slices, each a whole number of `unit` rows."""
        nu = rows // unit
        per = -(-nu // nthr)
        return [(i * per * unit, min(rows, (i + 1) * per * unit)) for i in range(nthr) if i * per < nu]

    x1 = inp.get("x:c1_per_tensor_s8")
    x2 = inp.get("x:c2_per_token_s8")
    w3 = inp.get("x:c3_per_group_u4_g128")
    xa = inp.get("x:c4_fp8_act_1x128")
    xw = inp.get("x:c4_fp8_weight_128x128")
    w5 = inp.get("x:c5_fp4_weight")
    g5 = np.float32(np.abs(oracle.widen(w5[:3584], "bf16")).max() / np.float32(2688.0))
    cases = [
        # name, sample, rows, row unit, algorithmic bytes, call(sample slice)
        ("per_tensor_s8", x1, 64, 64, x1.size * 5 + 4,
         lambda a: oracle.quant_int(a, "f32", "tensor", code="s8")),
        ("per_token_s8", x2[:2048], 2048, 1, 2048 * 4096 * 3 + 2048 * 4,
         lambda a: oracle.quant_int(a, "bf16", "token", code="s8")),
        ("per_group_u4_g128", w3[:2752], 2752, 1, 2752 * 4096 * 2 + 2752 * 2048 + 2752 * 32 * 5,
         lambda a: oracle.quant_int(a, "f16", "group", axis=1, group_size=128, code="u4", symmetric=False)),
        ("fp8_1x128", xa[:1024], 1024, 1, 1024 * 7168 * 3 + 1024 * 56 * 4,
         lambda a: oracle.quant_fp8_block(a, "bf16", 1, 128)),
        ("fp8_128x128", xw[:1792], 1792, 128, 1792 * 7168 * 3 + 14 * 56 * 4,
         lambda a: oracle.quant_fp8_block(a, "bf16", 128, 128)),
        ("nvfp4_static_global", w5[:3584], 3584, 1, 3584 * 4096 * 2 + 3584 * 2048 + 3584 * 256 + 4,
         lambda a: oracle.quant_fp4_block(a, "bf16", "nvfp4", static_global=g5)),
        ("mxfp4", w5[:3584], 3584, 1, 3584 * 4096 * 2 + 3584 * 2048 + 3584 * 128,
         lambda a: oracle.quant_fp4_block(a, "bf16", "mxfp4")),
    ]
    per = {}
    pool = ThreadPoolExecutor(max_workers=nthr)
    for name, a, rows, unit, nbytes, call in cases:
        log("cpu baseline:", name)
        a = np.ascontiguousarray(a)
        reps = 50 if name == "per_tensor_s8" else 1
        t1 = best(lambda: [call(a) for _ in range(reps)]) / reps
        slices = split(rows, unit)
        parts = [np.ascontiguousarray(a[r0:r1]) for r0, r1 in slices]
        if len(parts) > 1:
            tN = best(lambda: list(pool.map(call, parts)))
        else:
            tN = t1
        per[name] = {"sample": "first %d of %d rows" % (rows, inp.get(
            {"per_tensor_s8": "x:c1_per_tensor_s8", "per_token_s8": "x:c2_per_token_s8",
             "per_group_u4_g128": "x:c3_per_group_u4_g128", "fp8_1x128": "x:c4_fp8_act_1x128",
             "fp8_128x128": "x:c4_fp8_weight_128x128"}.get(name, "x:c5_fp4_weight")).shape[0]),
                     "bytes": nbytes, "single_GBps": round(nbytes / t1 / 1e9, 4),
                     "all_cores_GBps": round(nbytes / tN / 1e9, 4), "threads": len(parts)}
    pool.shutdown()
    head = per["per_token_s8"]
    return {"value": head["all_cores_GBps"], "unit": "GB/s", "cores": head["threads"], "kind": "oracle",
            "sample": "per-token s8 quantize of the first 2048 of 8192 rows of the bf16 [8192,4096] workload, "
                      "rows split over %d OS threads (one unchanged oracle call per slice), best of 3" % head["threads"],
            "single": head["single_GBps"], "cpu_model": model, "cpu_count": ncpu, "threads_available": avail,
            "per_config": per, "note": "the NVFP4 sample takes the per-tensor scale of the sample as a static "
                                       "input, so its rows split without a serial max pass"}


# ------------------------------------------------------------------ rocprofv3 summaries
def _csvs(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def trace_summary(d):
    """Per-kernel dispatch count, mean, median, p10, p90, min, max (us) from
    the rocprofv3 kernel-trace CSVs under `d`."""
    import numpy as np
    dur = {}
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            k = r.get("Kernel_Name") or r.get("Name")
            dur.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    rows = sorted(dur.items(), key=lambda kv: -sum(kv[1]))
    print("%-110s %6s %9s %9s %9s %9s %9s %9s" % ("kernel", "calls", "mean_us", "median", "p10", "p90", "min", "max"))
    for k, v in rows:
        a = np.array(v)
        print("%-110s %6d %9.2f %9.2f %9.2f %9.2f %9.2f %9.2f" % (
            k[:110], a.size, a.mean(), np.median(a), np.percentile(a, 10), np.percentile(a, 90), a.min(), a.max()))


def pmc_summary(d):
    """Per-kernel mean of every counter in the rocprofv3 counter CSVs under
    `d` (values per dispatch, summed over the dimensions rocprofv3 reports)."""
    acc = {}
    for f in _csvs(d, "counter_collection.csv"):
        per_dispatch = {}
        for r in csv.DictReader(open(f)):
            key = (r.get("Kernel_Name"), r["Counter_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        for (k, c, _), v in per_dispatch.items():
            acc.setdefault((k, c), []).append(v)
    print("%-110s %-22s %6s %16s" % ("kernel", "counter", "disp", "mean"))
    for (k, c), v in sorted(acc.items()):
        print("%-110s %-22s %6d %16.1f" % (k[:110], c, len(v), sum(v) / len(v)))


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every row, group and tile is "
              "independent, so the work shards without communication).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import tensor_quantization_amd as tq
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel(), "bytes_written": b.numel(), "launches": 10}))
        return
    inp = Inputs()
    if args.only:
        if args.only.startswith("quant_") and args.only[6:] in [o[0] for o in quantizers(torch, tq, inp)]:
            res, _, _ = run_quantizers(torch, tq, inp, args.steps, args.warmup, args.iters, only=args.only)
        elif args.only == "path":
            res = run_path(torch, tq, inp, args.steps)
        elif args.only.startswith("ceiling_"):
            c = [c for c in CEILINGS if c[0] == args.only[8:]][0]
            res = stream_ceiling(torch, tq, *c[1:], iters=args.iters)
        else:
            res = breakdown(torch, tq, inp, iters=args.iters, only=args.only)
        print(json.dumps(res))
        return
    log("quantize: per-token s8 bf16 [8192,4096], steps=%d warmup=%d" % (args.steps, args.warmup))
    quant, head, qceil = run_quantizers(torch, tq, inp, args.steps, args.warmup, args.iters)
    nbytes, wall, ev_us = head
    value = nbytes * args.steps / wall / 1e9
    q = quant["per_token_s8"]
    roofline = {"kernel": "quant_per_token_s8 (k_quant_rows)", "bound": "hbm", "achieved": q["GBps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": q["frac"], "traffic": read_traffic("quant_per_token_s8"),
                "algorithmic_bytes_per_launch": nbytes, "mean_launch_us": q["us"]}
    log("copy ceilings")
    ceilings = {c[0]: stream_ceiling(torch, tq, *c[1:], iters=args.iters) for c in CEILINGS}
    log("per-token path")
    path = run_path(torch, tq, inp, args.steps)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1000, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "per-token W8A8 quantize: bf16 [8192,4096] N(0,1), 1% outlier columns x20, "
                               "symmetric s8 [-127,127], one fp32 scale per row; step = one quantize launch",
                   "rows": 8192, "cols": 4096, "input": "bf16", "code": "s8", "bytes_per_step": nbytes,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "quantize": quant,
        "copy_ceiling": ceilings,
        "path": path,
    }
    if not args.no_breakdown:
        line["breakdown"] = breakdown(torch, tq, inp, iters=args.iters, ceil_cache=qceil)
    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        line["cpu_baseline"] = cpu_baseline(inp)
    line["inputs_sha256"] = inp.sha256()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
