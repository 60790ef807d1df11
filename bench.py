#!/usr/bin/env python3
"""Benchmark of the quantization hot path on one MI355X.

A step is one pass of the whole per-token path over the per-token W8A8
workload (bf16 [8192, 4096], N(0,1) with 1% outlier columns x20, symmetric
s8, one fp32 scale per row): quantize, dequantize to bf16, STE backward with
a bf16 dy, and dequantize backward.  `value` is the step's algorithmic bytes
(every input read once + every output written once) divided by the wall time
of K steps, in GB/s.  Inputs are resident in HBM before the timed region and
rotate over several buffer sets (more than 1 GB in total) so that the 256 MB
last-level cache cannot serve a repeat.

Also reported on the same JSON line:
  roofline      the dominant kernel of the step (most time): algorithmic
                bytes per launch / its mean launch time from HIP events on
                the launch stream, against the 8 TB/s HBM peak; `traffic` is
                the HBM bytes per launch measured by rocprofv3 counters
                (profiles/hbm_traffic_*.txt), null when the kernel source
                changed since that measurement.
  kernels       every kernel of the step with its own GB/s and HBM fraction.
  breakdown     the other workloads (per-tensor s8 f32 [64,256]; per-group u4
                g128 f16 [11008,4096]; FP8 1x128 bf16 [4096,7168]; FP8
                128x128 bf16 [7168,7168]; NVFP4 and MXFP4 bf16 [14336,4096]
                and their GEMM-layout transposes), each op timed alone.
  cpu_baseline  the CPU oracle (single thread) on full steps of the same
                workload, repeated for about 10 s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-breakdown]
       [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default=None, help="time one breakdown op (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy 10 times (scales the HBM byte counters)")
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


LLC_BYTES = 256 << 20


def nsets_for(read_bytes, set_bytes, cap_bytes=16 << 30):
    """Buffer sets to rotate so that a set's inputs are re-read only after at
    least twice the last-level cache of other reads (non-temporal stores do
    not allocate there, so reads alone must overflow it), and at least 1.2 GB
    in total; at most 64 sets (the tiny per-tensor workload is latency-bound
    and stays cache-resident) and cap_bytes of device memory."""
    n = max(4, -(-2 * LLC_BYTES // max(1, read_bytes)), -(-int(1.2e9) // max(1, set_bytes)))
    return max(2, min(n, 64, cap_bytes // max(1, set_bytes)))


def check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed with status %d" % (what, rc))


# The step's kernels (per-token quantize, dequantize, STE, dequantize
# backward) are built from these sources only; a counter summary taken from
# other versions of them is stale.
STEP_SOURCES = ("tq_int.hip", "tq_device.h", "tq_host.h")


def source_digest():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "tensor_quantization_amd", "csrc")
    for f in STEP_SOURCES:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.txt" % kernel)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ main step
def build_step(torch, tq):
    import numpy as np
    import workloads
    rows, cols = 8192, 4096
    x = workloads.make_input("c2_per_token_s8")
    dy = workloads.make_dy("c2_per_token_s8")
    L = tq._lib
    per_set = rows * cols * 2 * 5 + rows * cols + rows * 4
    nsets = nsets_for(rows * cols, per_set)        # smallest read stream: the s8 codes
    x0, dy0 = dev_bits(x, "bf16", torch), dev_bits(dy, "bf16", torch)
    sets = []
    for i in range(nsets):
        sets.append(dict(
            x=x0 if i == 0 else x0.clone(), dy=dy0 if i == 0 else dy0.clone(),
            q=torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
            s=torch.empty(rows, dtype=torch.float32, device="cuda"),
            y=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
            dx=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"),
            dq=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    BF16, S8 = 2, 0
    n = rows * cols
    kernels = {
        # name: (algorithmic bytes per launch, callable(set))
        "quant_per_token_s8": (n * 2 + n + rows * 4, lambda b: check(L.tq_quant_per_token(
            P(b["x"]), BF16, rows, cols, S8, -127, 127, P(b["q"]), P(b["s"]), None, stream), "quant")),
        "dequant_per_token_s8": (n + rows * 4 + n * 2, lambda b: check(L.tq_dequant_per_token(
            P(b["q"]), S8, rows, cols, P(b["s"]), None, P(b["y"]), BF16, stream), "dequant")),
        "quant_per_token_s8_backward": (n * 2 * 3 + rows * 4, lambda b: check(L.tq_quant_per_token_backward(
            P(b["x"]), BF16, rows, cols, S8, -127, 127, P(b["s"]), None, P(b["dy"]), P(b["dx"]), stream), "ste")),
        "dequant_per_token_backward": (n * 2 * 2 + rows * 4, lambda b: check(L.tq_dequant_per_token_backward(
            P(b["dy"]), BF16, rows, cols, P(b["s"]), P(b["dq"]), stream), "dqb")),
    }
    return sets, kernels


def run_step_bench(torch, tq, steps, warmup):
    """K steps, issued kernel by kernel: K quantize launches, then K dequantize,
    K STE backward and K dequantize backward launches -- the same work and
    dependency order as K whole steps.  One launch counter runs through all
    of them and picks the buffer set, so every launch reads the set touched
    longest ago (its inputs were last used nsets launches earlier).  One HIP
    event pair brackets each kernel's K back-to-back launches on the launch
    stream, so its mean launch time carries no per-launch event overhead."""
    sets, kernels = build_step(torch, tq)
    names = list(kernels)
    step_bytes = sum(kernels[k][0] for k in names)
    c = 0
    for i in range(warmup):
        for k in names:
            kernels[k][1](sets[c % len(sets)])
            c += 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    c = 0
    for j, k in enumerate(names):
        for i in range(steps):
            kernels[k][1](sets[c % len(sets)])
            c += 1
        ev[j + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = {}
    for j, k in enumerate(names):
        us = 1000.0 * ev[j].elapsed_time(ev[j + 1]) / steps
        gbps = kernels[k][0] / (us * 1e-6) / 1e9
        per_kernel[k] = {"bytes": kernels[k][0], "us": round(us, 3), "GBps": round(gbps, 1),
                         "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    return step_bytes, wall, per_kernel


# ------------------------------------------------------------------ breakdown
def breakdown(torch, tq, iters=20, only=None):
    import numpy as np
    import workloads
    L = tq._lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []

    def bench_op(name, cfg, nbytes, make_set, launch, set_bytes, read_bytes, flops=None, peak=FP8_PEAK_TFLOPS):
        if only and only != name:
            return
        log("breakdown:", name)
        sets = [make_set(i) for i in range(nsets_for(read_bytes, set_bytes))]
        for i in range(3):
            launch(sets[i % len(sets)])
        s_ev = torch.cuda.Event(enable_timing=True)
        e_ev = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s_ev.record()
        for i in range(iters):
            launch(sets[i % len(sets)])
        e_ev.record()
        torch.cuda.synchronize()
        us = 1000.0 * s_ev.elapsed_time(e_ev) / iters
        gbps = nbytes / (us * 1e-6) / 1e9
        if flops is None:
            out.append({"op": name, "workload": cfg, "bytes": nbytes, "us": round(us, 3), "GBps": round(gbps, 1),
                        "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        else:
            tf = flops / (us * 1e-6) / 1e12
            out.append({"op": name, "workload": cfg, "flops": flops, "us": round(us, 3), "TFLOPs": round(tf, 1),
                        "frac": round(tf / peak, 4), "bound": "mfma"})
        del sets
        torch.cuda.empty_cache()

    E = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    u8, f32, bf16, f16 = torch.uint8, torch.float32, torch.bfloat16, torch.float16

    # per-tensor s8, f32 [64, 256]
    x1 = workloads.make_input("c1_per_tensor_s8")
    dy1 = workloads.make_dy("c1_per_tensor_s8")
    n1 = x1.size
    mk1 = lambda i: dict(x=dev_bits(x1, "f32", torch), dy=dev_bits(dy1, "f32", torch), q=E(n1, u8), s=E(1, f32),
                         ws=E(8192, u8), y=E(n1, f32), dx=E(n1, f32))
    bench_op("quant_per_tensor_s8", "c1 f32 [64,256]", n1 * 4 + n1 + 4, mk1,
             lambda b: check(L.tq_quant_per_tensor(P(b["x"]), 0, n1, 0, -127, 127, 0, P(b["q"]), P(b["s"]), None,
                                                   P(b["ws"]), 8192, stream), "c1 quant"), n1 * 20, n1 * 4)
    bench_op("quant_per_tensor_s8_backward", "c1 f32 [64,256]", n1 * 12 + 4, mk1,
             lambda b: check(L.tq_quant_per_tensor_backward(P(b["x"]), 0, n1, 0, -127, 127, P(b["s"]), None,
                                                            P(b["dy"]), P(b["dx"]), stream), "c1 ste"), n1 * 20, n1 * 8)

    # per-tensor fake quantization (round trip) and its backward on the c2
    # activations bf16 [8192, 4096]: dynamic scale (reduce + round trip),
    # static scale (one pass), straight-through backward
    x2 = workloads.make_input("c2_per_token_s8")
    dy2 = workloads.make_dy("c2_per_token_s8")
    n2 = x2.size
    mkf2 = lambda i: dict(x=dev_bits(x2, "bf16", torch), dy=dev_bits(dy2, "bf16", torch), y=E(n2, bf16),
                          s=torch.full((1,), 0.03, dtype=f32, device="cuda"), ws=E(8192, u8), dx=E(n2, bf16))
    cfg2 = "c2 bf16 [8192,4096] per-tensor s8"
    bench_op("fake_quant_per_tensor_s8_dynamic", cfg2, n2 * 4 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor(P(b["x"]), 2, n2, 0, -127, 127, 0, P(b["y"]), P(b["s"]), None,
                                                        P(b["ws"]), 8192, stream), "fake dyn"), n2 * 8, n2 * 2)
    bench_op("fake_quant_per_tensor_s8_static", cfg2, n2 * 4 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor(P(b["x"]), 2, n2, 0, -127, 127, 1, P(b["y"]), P(b["s"]), None,
                                                        None, 0, stream), "fake static"), n2 * 8, n2 * 2)
    bench_op("fake_quant_per_tensor_s8_backward", cfg2, n2 * 6 + 4, mkf2,
             lambda b: check(L.tq_fake_quant_per_tensor_backward(P(b["x"]), 2, n2, 0, -127, 127, P(b["s"]), None,
                                                                 P(b["dy"]), P(b["dx"]), stream), "fake bwd"),
             n2 * 8, n2 * 4)

    # binary64 inputs: the per-token workload's shape in f64 (N(0,1) values)
    xf = np.random.default_rng(211).standard_normal((8192, 4096))
    shpf = (ctypes.c_int64 * 2)(8192, 4096)
    mkd = lambda i: dict(x=torch.from_numpy(xf).cuda(), q=E(n2, u8), s=E(8192, torch.float64),
                         y=E((8192, 4096), torch.float64))
    bench_op("quant_f64_per_token_s8", "f64 [8192,4096] per-token s8", n2 * 9 + 8192 * 8, mkd,
             lambda b: check(L.tq_quant_f64(P(b["x"]), 2, shpf, 2, 0, 0, 0, -127, 127, 0, P(b["q"]), P(b["s"]), None,
                                            None, 0, stream), "f64 quant"), n2 * 17, n2 * 8)
    bench_op("dequant_f64_per_token_s8", "f64 [8192,4096] per-token s8", n2 * 9 + 8192 * 8, mkd,
             lambda b: check(L.tq_dequant_f64(P(b["q"]), 0, 2, shpf, 2, 0, 0, P(b["s"]), None, P(b["y"]), stream),
                             "f64 dequant"), n2 * 17, n2)
    del xf

    # per-group u4 g128 asymmetric, f16 [11008, 4096]
    w3 = workloads.make_input("c3_per_group_u4_g128")
    N3, K3 = w3.shape
    n3 = w3.size
    shp3 = (ctypes.c_int64 * 2)(N3, K3)
    b3 = n3 * 2 + n3 // 2 + (n3 // 128) * 5
    mk3 = lambda i: dict(x=dev_bits(w3, "f16", torch), q=E((N3, K3 // 2), u8), s=E((N3, K3 // 128), f32),
                         z=E((N3, K3 // 128), u8), y=E((N3, K3), f16))
    bench_op("quant_per_group_u4_g128", "c3 f16 [11008,4096]", b3, mk3,
             lambda b: check(L.tq_quant_per_group(P(b["x"]), 1, 2, shp3, 1, 128, 3, 0, 15, P(b["q"]), P(b["s"]),
                                                  P(b["z"]), stream), "c3 quant"), b3 + n3 * 2, n3 * 2)
    bench_op("dequant_per_group_u4_g128", "c3 f16 [11008,4096]", b3, mk3,
             lambda b: check(L.tq_dequant_per_group(P(b["q"]), 3, 2, shp3, 1, 128, P(b["s"]), P(b["z"]), P(b["y"]),
                                                    1, stream), "c3 dequant"), b3 + n3 * 2, n3 // 2 + (n3 // 128) * 5)

    # FP8 1x128 activations bf16 [4096, 7168]; 128x128 weights bf16 [7168, 7168]
    for key, name in (("c4_fp8_act_1x128", "fp8_1x128"), ("c4_fp8_weight_128x128", "fp8_128x128")):
        xa = workloads.make_input(key)
        R, C = xa.shape
        br, bc = workloads.CONFIGS[key]["block"]
        ns = (R // br) * (C // bc)
        nb = R * C * 3 + ns * 4
        mk = lambda i, xa=xa, R=R, C=C, ns=ns: dict(x=dev_bits(xa, "bf16", torch), q=E((R, C), u8), s=E(ns, f32),
                                                    y=E((R, C), bf16))
        cfg = "c4 bf16 [%d,%d] %dx%d" % (R, C, br, bc)
        bench_op("quant_" + name, cfg, nb, mk,
                 lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_quant_fp8_block(P(b["x"]), 2, R, C, br, bc, P(b["q"]),
                                                                              P(b["s"]), stream), "fp8 quant"),
                 nb + R * C * 2, R * C * 2)
        bench_op("dequant_" + name, cfg, nb, mk,
                 lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_dequant_fp8_block(P(b["q"]), R, C, br, bc, P(b["s"]),
                                                                                P(b["y"]), 2, stream), "fp8 deq"),
                 nb + R * C * 2, R * C + ns * 4)
        if name == "fp8_1x128":     # dequantize backward (A9) on the activation shape: dq = dy * scale
            mkb = lambda i, R=R, C=C, ns=ns: dict(dy=dev_bits(xa, "bf16", torch), s=torch.ones(ns, dtype=f32, device="cuda"),
                                                  dq=E((R, C), bf16))
            bench_op("dequant_backward_" + name, cfg, R * C * 4 + ns * 4, mkb,
                     lambda b, R=R, C=C, br=br, bc=bc: check(L.tq_dequant_fp8_block_backward(
                         P(b["dy"]), 2, R, C, br, bc, P(b["s"]), P(b["dq"]), stream), "fp8 dqb"),
                     R * C * 4 + ns * 4, R * C * 2 + ns * 4)

    # MXFP8 on the c4 activations bf16 [4096, 7168]: E4M3 + E8M0 per 32
    xm = workloads.make_input("c4_fp8_act_1x128")
    Rm, Cm = xm.shape
    nm = xm.size
    bm = nm * 2 + nm + nm // 32
    mkm = lambda i: dict(x=dev_bits(xm, "bf16", torch), q=E((Rm, Cm), u8), b=E((Rm, Cm // 32), u8),
                         y=E((Rm, Cm), bf16))
    bench_op("quant_mxfp8", "c4 bf16 [4096,7168] MXFP8", bm, mkm,
             lambda b: check(L.tq_quant_mxfp8(P(b["x"]), 2, Rm, Cm, P(b["q"]), P(b["b"]), stream), "mxfp8"),
             bm + nm * 2, nm * 2)
    bench_op("dequant_mxfp8", "c4 bf16 [4096,7168] MXFP8", bm, mkm,
             lambda b: check(L.tq_dequant_mxfp8(P(b["q"]), P(b["b"]), Rm, Cm, P(b["y"]), 2, stream), "mxfp8 deq"),
             bm + nm * 2, nm + nm // 32)

    # FP4: NVFP4 (dynamic and static per-tensor scale), MXFP4, transposes
    w5 = workloads.make_input("c5_fp4_weight")
    N5, K5 = w5.shape
    n5 = w5.size
    for kind, gs in (("nvfp4", 16), ("mxfp4", 32)):
        nb = n5 * 2 + n5 // 2 + n5 // gs + (4 if kind == "nvfp4" else 0)
        mk = lambda i, gs=gs: dict(x=dev_bits(w5, "bf16", torch), p=E((N5, K5 // 2), u8), b=E((N5, K5 // gs), u8),
                                   g=torch.full((1,), 1.2e-5, dtype=f32, device="cuda"), ws=E(8192, u8),
                                   pt=E((K5 // 2, N5), u8), bt=E((K5 // gs, N5), u8))
        cfg = "c5 bf16 [14336,4096]"
        if kind == "nvfp4":
            bench_op("quant_nvfp4_dynamic_global", cfg, nb, mk,
                     lambda b: check(L.tq_quant_fp4_block(P(b["x"]), 2, N5, K5, 0, P(b["p"]), P(b["b"]), P(b["g"]), 0,
                                                          P(b["ws"]), 8192, stream), "nvfp4"), nb + n5, n5 * 2)
            bench_op("quant_nvfp4_static_global", cfg, nb, mk,
                     lambda b: check(L.tq_quant_fp4_block(P(b["x"]), 2, N5, K5, 0, P(b["p"]), P(b["b"]), P(b["g"]), 1,
                                                          None, 0, stream), "nvfp4 static"), nb + n5, n5 * 2)
        else:
            bench_op("quant_mxfp4", cfg, nb, mk,
                     lambda b: check(L.tq_quant_fp4_block(P(b["x"]), 2, N5, K5, 1, P(b["p"]), P(b["b"]), None, 1,
                                                          None, 0, stream), "mxfp4"), nb + n5, n5 * 2)
        # dequantize -> bf16 (A7 on the c5 weight): valid E2M1 codes, block scales of 1 (E4M3 0x38 / E8M0 127)
        mkd = lambda i, gs=gs, kind=kind: dict(
            p=torch.randint(0, 256, (N5, K5 // 2), dtype=u8, device="cuda"),
            b=torch.full((N5, K5 // gs), 0x38 if kind == "nvfp4" else 127, dtype=u8, device="cuda"),
            g=torch.full((1,), 1.2e-5, dtype=f32, device="cuda"), y=E((N5, K5), bf16))
        db = n5 // 2 + n5 // gs + (4 if kind == "nvfp4" else 0) + n5 * 2
        bench_op("dequant_" + kind, cfg, db, mkd,
                 lambda b, kd=(0 if kind == "nvfp4" else 1): check(
                     L.tq_dequant_fp4_block(P(b["p"]), P(b["b"]), P(b["g"]) if kd == 0 else None, N5, K5, kd,
                                            P(b["y"]), 2, stream), "fp4 dequant"),
                 db, n5 // 2 + n5 // gs)
        if kind == "nvfp4":         # dequantize backward (A9) on the weight shape: dq = dy * eff
            mkq = lambda i, gs=gs: dict(dy=dev_bits(w5, "bf16", torch), b=torch.full((N5, K5 // gs), 0x38, dtype=u8,
                                                                                     device="cuda"),
                                        g=torch.full((1,), 1.2e-5, dtype=f32, device="cuda"), dq=E((N5, K5), bf16))
            qb = n5 * 4 + n5 // gs + 4
            bench_op("dequant_backward_nvfp4", cfg, qb, mkq,
                     lambda b: check(L.tq_dequant_fp4_block_backward(P(b["dy"]), 2, P(b["b"]), P(b["g"]), N5, K5, 0,
                                                                      P(b["dq"]), stream), "nvfp4 dqb"),
                     qb, n5 * 2 + n5 // gs)
        tb = 2 * (n5 // 2 + n5 // gs)
        bench_op("transpose_for_gemm_" + kind, cfg, tb, mk,
                 lambda b, gs=gs: check(L.tq_fp4_transpose_for_gemm(P(b["p"]), P(b["b"]), N5, K5, gs, P(b["pt"]),
                                                                    P(b["bt"]), stream), "transpose"),
                 nb + n5, tb // 2)

    # FP4 layout follow-ons on the NVFP4 c5 weight: gate + up fused into one
    # [2048, 28672] GEMM operand, the two stacked by rows, and the FP8 expansion
    pb, sbb = n5 // 2, n5 // 16
    mkf = lambda i: dict(p1=E((N5, K5 // 2), u8), b1=E((N5, K5 // 16), u8), p2=E((N5, K5 // 2), u8),
                         b2=E((N5, K5 // 16), u8), pt=E((K5 // 2, 2 * N5), u8), bt=E((K5 // 16, 2 * N5), u8),
                         po=E((2 * N5, K5 // 2), u8), bo=E((2 * N5, K5 // 16), u8), f8=E((N5, K5), u8))
    cfg = "c5 nvfp4 2 x [14336,4096]"

    def concat_t(b):
        pp = (ctypes.c_void_p * 2)(b["p1"].data_ptr(), b["p2"].data_ptr())
        bb = (ctypes.c_void_p * 2)(b["b1"].data_ptr(), b["b2"].data_ptr())
        nn = (ctypes.c_int64 * 2)(N5, N5)
        check(L.tq_fp4_transpose_concat_for_gemm(2, pp, bb, nn, K5, 16, 128, P(b["pt"]), P(b["bt"]), None,
                                                 stream), "transpose concat")
    bench_op("transpose_concat_for_gemm_nvfp4", cfg, 4 * (pb + sbb), mkf, concat_t, 8 * (pb + sbb) + n5,
             2 * (pb + sbb))
    bench_op("concat_rows_nvfp4", cfg, 4 * (pb + sbb), mkf,
             lambda b: check(L.tq_fp4_concat_rows(P(b["p1"]), P(b["b1"]), 1.5e-5, P(b["p2"]), P(b["b2"]), 1.5e-5, N5,
                                                  N5, K5, P(b["po"]), P(b["bo"]), stream), "concat rows"),
             8 * (pb + sbb) + n5, 2 * (pb + sbb))
    bench_op("predequant_to_fp8_nvfp4", "c5 nvfp4 [14336,4096]", pb + sbb + n5, mkf,
             lambda b: check(L.tq_fp4_predequant_to_fp8(P(b["p1"]), P(b["b1"]), 1.5e-5, N5, K5, 0, P(b["f8"]),
                                                        stream), "predequant"),
             8 * (pb + sbb) + n5, pb + sbb)

    # block-scaled FP8 GEMM: the c4 activations [4096, 7168] (1 x 128) times the
    # c4 weight [7168, 7168] (128 x 128), bf16 out; 2 M N K flops on the fp8 peak
    if not only or only == "fp8_block_gemm":
        Mg, Kg = 4096, 7168
        Ng = Kg
        xa = torch.from_numpy(workloads.make_input("c4_fp8_act_1x128").view(np.int16)).view(bf16).cuda()
        xw = torch.from_numpy(workloads.make_input("c4_fp8_weight_128x128").view(np.int16)).view(bf16).cuda()
        qa0, sa0 = tq.tq_quant_fp8_block(xa, 1, 128)
        qw0, sw0 = tq.tq_quant_fp8_block(xw, 128, 128)
        del xa, xw
        mkg = lambda i: dict(qa=qa0.clone(), sa=sa0.clone(), qw=qw0.clone(), sw=sw0.clone(), y=E((Mg, Ng), bf16))
        gb = Mg * Kg + Ng * Kg + 2 * Mg * Ng + 4 * (Mg * Kg // 128 + Ng * Kg // 16384)
        bench_op("fp8_block_gemm", "c4 fp8 [4096,7168] x [7168,7168]^T bf16 out", gb, mkg,
                 lambda b: check(L.tq_fp8_block_gemm(P(b["qa"]), P(b["sa"]), P(b["qw"]), P(b["sw"]), Mg, Ng, Kg,
                                                     P(b["y"]), 2, stream), "fp8 gemm"),
                 gb, Mg * Kg + Ng * Kg, flops=2 * Mg * Ng * Kg)
        del qa0, sa0, qw0, sw0

    # W8A8 quantized linear: the per-token s8 activations bf16 [8192, 4096]
    # times the f16 weight [11008, 4096] quantized per channel to s8, bf16 out
    if not only or only == "w8a8_linear":
        Mq, Kq, Nq = 8192, 4096, 11008
        xq = torch.from_numpy(workloads.make_input("c2_per_token_s8").view(np.int16)).view(bf16).cuda()
        wq = torch.from_numpy(workloads.make_input("c3_per_group_u4_g128").view(np.int16)).view(f16).cuda()
        qx0, sx0, _ = tq.tq_quant_per_token(xq)
        qw0, sw0, _ = tq.tq_quant_per_token(wq)
        del xq, wq
        mkq = lambda i: dict(qx=qx0.clone(), sx=sx0.clone(), qw=qw0.clone(), sw=sw0.clone(), y=E((Mq, Nq), bf16))
        qb = Mq * Kq + Nq * Kq + 2 * Mq * Nq + 4 * (Mq + Nq)
        bench_op("w8a8_linear", "c2 s8 [8192,4096] x c3 s8 [11008,4096]^T bf16 out", qb, mkq,
                 lambda b: check(L.tq_w8a8_linear(P(b["qx"]), P(b["sx"]), P(b["qw"]), P(b["sw"]), Mq, Nq, Kq,
                                                  P(b["y"]), 2, stream), "w8a8"),
                 qb, Mq * Kq + Nq * Kq, flops=2 * Mq * Nq * Kq)
        del qx0, sx0, qw0, sw0

    # FP4 weight-only linear: bf16 activations [8192, 4096] (the activation
    # workload's shape and recipe) times the NVFP4 weight [14336, 4096], bf16
    # out; the products run on the bf16 matrix cores
    if not only or only == "fp4_linear_nvfp4":
        Mf, Kf, Nf = 8192, 4096, 14336
        xf0 = torch.from_numpy(workloads.make_input("c2_per_token_s8").view(np.int16)).view(bf16).cuda()
        wf = torch.from_numpy(workloads.make_input("c5_fp4_weight").view(np.int16)).view(bf16).cuda()
        pf0, bf0, gf0 = tq.tq_quant_fp4_block(wf, "nvfp4")
        del wf
        mkf4 = lambda i: dict(x=xf0.clone(), p=pf0.clone(), b=bf0.clone(), g=gf0.clone(), y=E((Mf, Nf), bf16))
        fb4 = Mf * Kf * 2 + Nf * Kf // 2 + Nf * Kf // 16 + 2 * Mf * Nf
        bench_op("fp4_linear_nvfp4", "bf16 [8192,4096] x c5 nvfp4 [14336,4096]^T bf16 out", fb4, mkf4,
                 lambda b: check(L.tq_fp4_linear(P(b["x"]), 2, P(b["p"]), P(b["b"]), P(b["g"]), 0, Mf, Nf, Kf,
                                                 P(b["y"]), 2, stream), "fp4 linear"),
                 fb4, Mf * Kf * 2 + Nf * Kf // 2, flops=2 * Mf * Nf * Kf, peak=BF16_PEAK_TFLOPS)
        del xf0, pf0, bf0, gf0
    return out


# ------------------------------------------------------------------ CPU
def cpu_baseline(min_seconds=10.0):
    import numpy as np
    import oracle
    import workloads
    x = workloads.make_input("c2_per_token_s8")
    dy = workloads.make_dy("c2_per_token_s8")
    rows, cols = x.shape
    n = x.size
    step_bytes = (n * 2 + n + rows * 4) + (n + rows * 4 + n * 2) + (n * 6 + rows * 4) + (n * 4 + rows * 4)
    oracle.lib()
    reps, t = 0, 0.0
    while t < min_seconds and reps < 20:
        t0 = time.perf_counter()
        q, s, _ = oracle.quant_int(x, "bf16", "token", code="s8")
        oracle.dequant_int(q, "s8", x.shape, "token", scale=s, yt="bf16")
        oracle.quant_int_backward(x, "bf16", "token", code="s8", scale=s, dy=dy)
        oracle.dequant_int_backward(dy, "bf16", "token", scale=s)
        t += time.perf_counter() - t0
        reps += 1
    return {"value": round(step_bytes * reps / t / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full steps of the per-token workload (quantize, dequantize, STE backward, dequantize "
                      "backward on bf16 [8192,4096]), single-threaded scalar C, %.1f s" % (reps, t)}


def main():
    args = parse()
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
    log("step benchmark: per-token s8 path, bf16 [8192,4096], steps=%d warmup=%d" % (args.steps, args.warmup))
    if args.only:
        print(json.dumps(breakdown(torch, tq, only=args.only)))
        return
    step_bytes, wall, per_kernel = run_step_bench(torch, tq, args.steps, args.warmup)
    value = step_bytes * args.steps / wall / 1e9
    def roof(k):
        d = per_kernel[k]
        return {"kernel": k, "bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": d["frac"], "traffic": read_traffic(k), "algorithmic_bytes_per_launch": d["bytes"],
                "mean_launch_us": d["us"]}
    dom = max(per_kernel, key=lambda k: per_kernel[k]["us"])
    roofline = roof(dom)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1000, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "per-token W8A8 s8: bf16 [8192,4096] N(0,1), 1% outlier columns x20, symmetric "
                               "s8 [-127,127], fp32 scale per row; step = quantize + dequantize(bf16) + STE "
                               "backward(bf16 dy) + dequantize backward",
                   "rows": 8192, "cols": 4096, "input": "bf16", "code": "s8", "step_bytes": step_bytes,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "roofline_quantize": roof("quant_per_token_s8"),
        "kernels": per_kernel,
    }
    if not args.no_breakdown:
        line["breakdown"] = breakdown(torch, tq)
    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
