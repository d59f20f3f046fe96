#!/usr/bin/env python3
"""Throughput of the fused add-RMSNorm + SwiGLU(+FP8) kernels on one MI355X.

One step = one pass of the Qwen2.5-1.5B-shaped prefill layer's memory-bound
ops over 4,096 tokens: fused_add_rmsnorm on bf16 [4096, 1536] followed by
swiglu on bf16 gate_up [4096, 17920] -> [4096, 8960].  ``value`` is the
effective HBM bandwidth of the step: the algorithmic bytes (every input read
once, every output written once, the weight once) divided by the wall time of
K back-to-back steps with the inputs already resident in HBM.  Each op
rotates through buffer sets covering three times the 256 MB last-level
cache, so that every step reads HBM rather than that cache.

Beside every kernel the same rotation of buffers is also streamed by a plain
copy (libaarms_refcopy.so) that reads and writes exactly the same bytes with
no arithmetic, one 16-byte vector of each input per lane: ``of_ref_copy`` is
that copy's time over the kernel's (above 1: the kernel is faster).  It is a
reference, not a bound: the bound is the 8 TB/s HBM peak, and kernels that
issue their accesses differently can beat the copy.  ``--copy-sweep`` times
other designs of such copies instead (vectors per lane, grid-stride or
one-shot grids, streaming hints), and pure reads, pure writes and a 1:1 copy
of 1 GiB, and prints them as the JSON line.

The same run also measures, as supplementary figures, the static-FP8 SwiGLU
on Llama-70B's [8192, 57344] gate_up, the dynamic-FP8 norm on Llama-405B's
[2048, 16384] rows, the 16-token norm, the 28-layer decode chain under a
HIP graph, the rest of the quantisation matrix at the same shapes (rmsnorm
without the residual add, the static-scale and per-token E4M3 forms, MXFP4,
NVFP4 and per-128-value E4M3), one GPU's share of both Llama layers under
8-way sharding, and the start-up tuner's report; and it times the CPU
oracle on the host's cores on the headline workload (a baseline, not a
target).  --configs restricts the supplementary figures to matching keys.

Prints exactly one JSON line.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (10^9 B/s)
METRIC = "effective HBM GB/s and % of MI355X peak, fused add-RMSNorm + SwiGLU(+fp8)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip start-up tuning: the headline runs the library's heuristic variants")
    ap.add_argument("--no-autotune-report", action="store_true",
                    help="skip the tuner report over the supplementary shapes")
    ap.add_argument("--variants", default=None,
                    help="headline variants by name, 'norm=<name>;swiglu=<name>' (no tuning): to "
                         "profile the configuration a tuned run chose")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--configs", default=None,
                    help="regular expression: time only the supplementary measurements whose key "
                         "matches (the headline always runs); for counter passes over a few kernels")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--copy-sweep", action="store_true",
                    help="instead of the workloads, time plain copy designs (vectors per lane, one-shot or "
                         "grid-stride grid, streaming hints) at the read/write mixes and sizes of the "
                         "headline kernels and the Llama norm and SwiGLU, and pure reads, pure writes "
                         "and a 1:1 copy of 1 GiB; prints them as the JSON line")
    ap.add_argument("--phase-timeline", action="store_true",
                    help="instead of the workloads, record the per-wave phase timeline of the Llama-405B "
                         "per-token E4M3 norm (libaarms_stamps.so) and print its summary as the JSON line")
    return ap.parse_args()


# ----------------------------------------------------------------- bytes

def norm_bytes(T, H, quant=False):
    """x, residual read; residual_out written; out written (bf16 or fp8);
    weight read once; per-token scales written."""
    io = T * H * 2 * 3 + (T * H * (1 if quant else 2))
    return io + H * 2 + (T * 4 if quant else 0)


def swiglu_bytes(T, N, quant=False):
    return T * 2 * N * 2 + T * N * (1 if quant else 2) + (4 if quant else 0)


# ----------------------------------------------------------------- timing

def progress(*what):
    """A progress line on stderr (the JSON line goes to stdout)."""
    print("[bench]", *what, file=sys.stderr, flush=True)


class Timer:
    def __init__(self, torch):
        self.torch = torch

    def region(self, fn, reps):
        t = self.torch
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / reps  # ms per rep


    def warm(self, fn, seconds=0.1):
        """Launch fn until about `seconds` of device time have passed: after
        the host has left the GPU idle (input generation) its clocks take some
        tens of milliseconds of load to settle."""
        t = self.torch
        n = 0
        t0 = time.perf_counter()
        while True:
            for _ in range(20):
                fn(n)
                n += 1
            t.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


MALL_BYTES = 256e6             # MI355X last-level (Infinity) cache


def rotation_sets(bytes_per_launch):
    """Buffer sets to rotate so that one cycle touches >= 3x the LLC (at
    only 2x, some variants measured faster from what the LLC still held)."""
    import math
    return max(2, math.ceil(3 * MALL_BYTES / bytes_per_launch))


def traffic_from_profiles(kernel_key: str, src_hash: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources; else None."""
    for path in glob.glob(os.path.join(ROOT, "profiles", "*counters*.md")):
        with open(path) as f:
            txt = f.read()
        if ("kernel_sources_sha256: " + src_hash) not in txt:
            continue
        for line in txt.splitlines():
            if line.startswith("traffic_bytes_per_launch[" + kernel_key + "]:"):
                return float(line.split(":", 1)[1].split()[0])
    return None


def load_refcopy():
    """libaarms_refcopy.so: the plain streaming copies (built with the library)."""
    import ctypes as C
    from activation_add_rmsnorm_amd import _build
    if not os.path.exists(_build.REFCOPY_PATH):
        _build.build()
    lib = C.CDLL(_build.REFCOPY_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
    lib.aarms_reference_copy.argtypes = [vp, i32, vp, i32, vp, vp, i64, vp]
    lib.aarms_copy_design.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, i64, vp]
    lib.aarms_copy_held.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
    return lib


def refcopy_entry(kernel_us, copy_us, nbytes):
    return {"ref_copy_us": round(copy_us, 2),
            "ref_copy_GB/s": round(nbytes / (copy_us * 1e-6) / 1e9, 1),
            "of_ref_copy": round(copy_us / kernel_us, 3)}


def kernel_sources_hash():
    """Hash of the sources of the library's kernels and their launch code
    (not of the reference copy, which no counter summary measures)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "activation_add_rmsnorm_amd", "csrc", "*"))):
        if os.path.basename(p) == "refcopy.hip":
            continue
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the kernels are row-independent and the library "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_add_rmsnorm_amd as A
    from workloads import configs as W

    lib = A.load()
    clib = load_refcopy()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    timer = Timer(torch)
    if args.copy_sweep:
        print(json.dumps(copy_sweep(args, torch, clib, dev, sp, timer)), flush=True)
        return
    if args.phase_timeline:
        print(json.dumps(phase_timeline(args, torch, np, W, dev, sp, timer)), flush=True)
        return

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ------------------------------------------------------------ headline
    wn, ws = W.NORM_PREFILL4096, W.SWIGLU_PREFILL4096
    T, H, N = wn.tokens, wn.hidden, ws.inter
    nd = W.norm_inputs(wn)
    gd = W.swiglu_inputs(ws)
    x0, r0, w0, gu0 = to_dev(nd["x"]), to_dev(nd["residual"]), to_dev(nd["weight"]), to_dev(gd["gate_up"])
    step_bytes_norm = norm_bytes(T, H)
    step_bytes_swiglu = swiglu_bytes(T, N)
    step_bytes = step_bytes_norm + step_bytes_swiglu
    # Separate rotation pools for the two ops, each cycling through at least
    # three times the 256 MB last-level cache, so that every launch -- in the step
    # loop and in the per-kernel loops -- reads HBM.
    n_norm = rotation_sets(step_bytes_norm)
    n_sw = rotation_sets(step_bytes_swiglu)
    norm_sets, sw_sets = [], []
    for _ in range(n_norm):
        s = dict(x=x0.clone(), r=r0.clone(), out=torch.empty_like(x0), ro=torch.empty_like(r0))
        s["p"] = (s["out"].data_ptr(), s["ro"].data_ptr(), s["x"].data_ptr(), s["r"].data_ptr(),
                  w0.data_ptr())
        norm_sets.append(s)
    for _ in range(n_sw):
        s = dict(gu=gu0.clone(), y=torch.empty((T, N), dtype=torch.bfloat16, device=dev))
        s["p"] = (s["y"].data_ptr(), s["gu"].data_ptr())
        sw_sets.append(s)
    eps = wn.eps

    # Start-up tuning (before any timed region): every variant that fits is
    # timed on this device at the headline shapes, and one is installed only
    # if it beats the library's heuristic choice by more than 3%; the step is
    # then timed with the installed variants (-1: the heuristic's), and once
    # more with the heuristic's alone for comparison.
    from activation_add_rmsnorm_amd import tuning
    tune_report = None
    if args.variants:
        given = dict(kv.split("=", 1) for kv in args.variants.split(";"))
        by_name = lambda op, n: [v for v in range(A.variant_count(op)) if A.variant_name(op, v) == n][0]
        variant = {"norm": by_name(A.OP_NORM, given["norm"]), "swiglu": by_name(A.OP_SWIGLU, given["swiglu"])}
    else:
        if not args.no_tune:
            tune_report = [tuning.tune("fused_add_rmsnorm", T, H), tuning.tune("swiglu", T, N)]
        variant = {"norm": tuning.variant_for("fused_add_rmsnorm", T, H),
                   "swiglu": tuning.variant_for("swiglu", T, N)}

    def norm_call(i, v=None):
        st = lib.fused_add_rmsnorm_ex(*norm_sets[i % n_norm]["p"], T, H, eps,
                                      variant["norm"] if v is None else v, sp)
        if st:
            raise A.AarmsError(st, "fused_add_rmsnorm")

    def swiglu_call(i, v=None):
        st = lib.swiglu_ex(*sw_sets[i % n_sw]["p"], T, N, variant["swiglu"] if v is None else v, sp)
        if st:
            raise A.AarmsError(st, "swiglu")

    def step(i):
        norm_call(i)
        swiglu_call(i)

    def step_heuristic(i):
        norm_call(i, -1)
        swiglu_call(i, -1)

    def stream(*a):
        st = clib.aarms_reference_copy(*a, sp)
        if st:
            raise RuntimeError("aarms_reference_copy: %d" % st)

    def norm_refcopy(i):
        s = norm_sets[i % n_norm]
        stream(s["ro"].data_ptr(), 16, s["out"].data_ptr(), 16, s["x"].data_ptr(), s["r"].data_ptr(), T * H // 8)

    def swiglu_refcopy(i):
        s = sw_sets[i % n_sw]
        gu = s["gu"].data_ptr()
        stream(s["y"].data_ptr(), 16, None, 0, gu, gu + T * N * 2, T * N // 8)

    K, Wu = args.steps, args.warmup
    progress("headline step")
    # ~50 ms of the step first, so that the clocks have settled from the host
    # work before (input generation; with --no-tune nothing else has run)
    # whatever W is; then the W warm-up steps right before the timed K
    timer.warm(step, 0.05)
    for i in range(Wu):
        step(i)
    ms_step = timer.region(step, K)
    if variant["norm"] == -1 and variant["swiglu"] == -1:
        ms_step_heuristic = ms_step
    else:
        timer.warm(step_heuristic, 0.02)
        ms_step_heuristic = timer.region(step_heuristic, K)

    # per-kernel durations: each kernel alone, back-to-back launches over
    # the same rotation, HIP events on the launch stream at both ends
    # (at least 200 launches each, whatever K: a region of a few launches
    # carries the events' own overhead)
    Kk = max(K, 200)
    norm_us = timer.region(norm_call, Kk) * 1e3
    swiglu_us = timer.region(swiglu_call, Kk) * 1e3
    timer.warm(norm_refcopy, 0.02)
    norm_copy_us = timer.region(norm_refcopy, Kk) * 1e3
    timer.warm(swiglu_refcopy, 0.02)
    swiglu_copy_us = timer.region(swiglu_refcopy, Kk) * 1e3

    value = step_bytes / (ms_step * 1e-3) / 1e9
    src_hash = kernel_sources_hash()
    roof = {
        "bound": "hbm",
        "kernel": "swiglu [4096,17920]->[4096,8960]",
        "achieved": round(step_bytes_swiglu / (swiglu_us * 1e-6) / 1e9, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
    }
    roof["frac"] = round(roof["achieved"] / HBM_PEAK_GBS, 4)
    roof["traffic"] = traffic_from_profiles("swiglu_qwen_prefill4096", src_hash)
    roof["bytes_per_launch"] = step_bytes_swiglu
    roof["avg_launch_us"] = round(swiglu_us, 2)
    roof.update(refcopy_entry(swiglu_us, swiglu_copy_us, step_bytes_swiglu))

    extra = {
        "norm_4096x1536": {"bytes": step_bytes_norm, "avg_launch_us": round(norm_us, 2),
                           "GB/s": round(step_bytes_norm / (norm_us * 1e-6) / 1e9, 1),
                           **refcopy_entry(norm_us, norm_copy_us, step_bytes_norm)},
        "swiglu_4096x17920": {"bytes": step_bytes_swiglu, "avg_launch_us": round(swiglu_us, 2),
                              "GB/s": roof["achieved"],
                              **refcopy_entry(swiglu_us, swiglu_copy_us, step_bytes_swiglu)},
        "buffer_sets_rotated": {"norm": n_norm, "swiglu": n_sw},
    }
    for k, tkey, nb in (("norm_4096x1536", "norm_qwen_prefill4096", step_bytes_norm),
                        ("swiglu_4096x17920", "swiglu_qwen_prefill4096", step_bytes_swiglu)):
        t = traffic_from_profiles(tkey, src_hash)
        if t is not None:
            extra[k]["traffic_bytes_per_launch"] = t
            extra[k]["traffic_over_algorithmic"] = round(t / nb, 4)
    name = lambda op, v, T_, W_, q: A.variant_name(op, v if v >= 0 else A.pick_variant(op, T_, W_, q))
    headline_variants = {
        "norm": name(A.OP_NORM, variant["norm"], T, H, False),
        "swiglu": name(A.OP_SWIGLU, variant["swiglu"], T, N, 0),
        "chosen_by": ("given (--variants)" if args.variants else
                      "start-up tuning" if (variant["norm"] >= 0 or variant["swiglu"] >= 0) else "heuristic"),
        "heuristic": {"norm": name(A.OP_NORM, -1, T, H, False), "swiglu": name(A.OP_SWIGLU, -1, T, N, 0),
                      "ms_per_step": round(ms_step_heuristic, 5),
                      "GB/s": round(step_bytes / (ms_step_heuristic * 1e-3) / 1e9, 1)},
        "tuning": tune_report,
    }
    tuning.clear()
    del norm_sets, sw_sets, x0, r0, gu0
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ supplementary
    configs = {}
    if not args.no_extra:
        configs = supplementary(args, torch, np, A, lib, clib, W, dev, sp, timer, to_dev)

    # ------------------------------------------------------------ cpu baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, W, nd, gd, step_bytes, args.cpu_seconds)

    if args.calibrate_copy:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic (seeded normals, Qwen2.5-1.5B prefill-layer shapes; no weights)",
        "config": {
            "workload": "qwen1.5b_prefill4096: fused_add_rmsnorm bf16 [4096,1536] eps 1e-6 + "
                        "swiglu bf16 gate_up [4096,17920] -> [4096,8960]",
            "bytes_per_step": step_bytes,
            "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "variants": headline_variants,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": extra,
        "configs": configs,
        "device": torch.cuda.get_device_name(dev),
        "kernel_sources_sha256": src_hash,
    }
    print(json.dumps(line), flush=True)


# Read/write mixes of the copy sweep: (name, kind of aarms_copy_design,
# bytes per input vector pair moved, the workload whose mix and size it is).
COPY_MIXES = [
    ("swiglu_mix_220MB", 0, 48, "swiglu bf16 [4096,17920] -> [4096,8960]: two inputs, one output", 220200960),
    ("norm_mix_50MB", 1, 64, "fused_add_rmsnorm bf16 [4096,1536]: two inputs, two outputs", 50331648),
    ("norm_fp8_mix_235MB", 2, 56, "fused_add_rmsnorm_quant_fp8 [2048,16384]: two inputs, a bf16 and an e4m3 output",
     234881024),
    ("swiglu_fp8_mix_1174MB", 6, 40,
     "swiglu_quant_fp8 [8192,57344] -> e4m3 [8192,28672]: two inputs, an output of a quarter of their bytes",
     1174405120),
    ("read_only_1GB", 3, 32, "reads only (two inputs, no output)", 1 << 30),
    ("read_only_134MB", 3, 32, "reads only: the inputs of fused_add_rmsnorm_quant_fp8 [2048,16384]", 134217728),
    ("write_only_101MB", 4, 16, "writes only: the outputs of fused_add_rmsnorm_quant_fp8 [2048,16384]", 100663296),
    ("read_only_25MB", 3, 32, "reads only: the inputs of fused_add_rmsnorm [4096,1536]", 25165824),
    ("write_only_25MB", 4, 16, "writes only: the outputs of fused_add_rmsnorm [4096,1536]", 25165824),
    ("write_only_1GB", 4, 16, "writes only (one output, no input)", 1 << 30),
    ("copy_1GB", 5, 32, "one input, one output of the same bytes", 1 << 30),
]


def copy_sweep(args, torch, clib, dev, sp, timer):
    """Plain copies at the read/write mix and size of each headline kernel,
    pure reads, pure writes and a 1:1 copy at 1 GiB (what the device's HBM
    gives each direction alone), pure reads and pure writes of the Llama-405B
    and headline norms' inputs and outputs, and a copy of the headline norm's
    bytes in its layout with its stores held for a range of holds: 1, 2 or 4 vectors per lane, a one-shot grid or a
    grid-stride loop over two 4-wave blocks per CU, with and without the streaming
    hints; rotated buffer sets (3x the last-level cache) as in the workload
    measurements.  Median of 5 timed regions per design, designs interleaved."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    reps = max(20, args.steps // 2)
    out = {"metric": "plain copy designs: GB/s by read/write mix and size", "unit": "GB/s",
           "hbm_peak_GB/s": HBM_PEAK_GBS, "compute_units": cus, "mixes": {}}
    for name, kind, pair_bytes, what, nbytes in COPY_MIXES:
        n = nbytes // pair_bytes
        ns = rotation_sets(n * pair_bytes)
        sets = []
        for _ in range(ns):
            a = torch.empty(n * 16, dtype=torch.uint8, device=dev)
            b = torch.empty(n * 16, dtype=torch.uint8, device=dev)
            o0 = torch.empty(n * 16, dtype=torch.uint8, device=dev)
            o1 = torch.empty(n * (16 if kind == 1 else 8), dtype=torch.uint8, device=dev) if kind in (1, 2) else None
            sets.append((a, b, o0, o1))
        designs = [(u, grid, nt) for u in (1, 2, 4) for grid in ("one-shot", "grid-stride") for nt in (1, 0)]
        times = {d: [] for d in designs}
        for _ in range(5):
            for d in designs:
                u, grid, nt = d
                gb = 0 if grid == "one-shot" else cus * 2   # two 4-wave blocks (8 waves) per CU

                def call(i, u=u, gb=gb, nt=nt):
                    a, b, o0, o1 = sets[i % ns]
                    st = clib.aarms_copy_design(kind, u, nt, gb, o0.data_ptr(), o1.data_ptr() if o1 is not None else None,
                                                a.data_ptr(), b.data_ptr(), n, sp)
                    if st:
                        raise RuntimeError("aarms_copy_design: %d" % st)
                timer.warm(call, 0.02)
                times[d].append(timer.region(call, reps) * 1e3)
        rows = []
        for d in designs:
            us = sorted(times[d])[2]
            rows.append({"vectors_per_lane": d[0], "grid": d[1], "streaming_hints": bool(d[2]),
                         "us": round(us, 2), "GB/s": round(n * pair_bytes / (us * 1e-6) / 1e9, 1)})
        rows.sort(key=lambda r: r["us"])
        out["mixes"][name] = {"what": what, "bytes": n * pair_bytes, "buffer_sets_rotated": ns, "designs": rows}
        del sets
        torch.cuda.empty_cache()
    # the headline norm's layout (one wave per 1,536-wide row, 4,096 rows, all
    # resident), its stores held on the real-time clock for a range of holds
    T, row_vecs = 4096, 1536 // 8
    nb = T * row_vecs * 16
    ns = rotation_sets(4 * nb)
    sets = [tuple(torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(4)) for _ in range(ns)]
    holds = [0, 250, 280, 300, 320, 340, 360, 400]
    times = {h: [] for h in holds}
    for _ in range(5):
        for h in holds:
            def call(i, h=h):
                a, b, o0, o1 = sets[i % ns]
                st = clib.aarms_copy_held(T, row_vecs, h, o0.data_ptr(), o1.data_ptr(), a.data_ptr(), b.data_ptr(), sp)
                if st:
                    raise RuntimeError("aarms_copy_held: %d" % st)
            timer.warm(call, 0.02)
            times[h].append(timer.region(call, max(reps, 200)) * 1e3)
    out["norm_layout_held_copy_50MB"] = {
        "what": "fused_add_rmsnorm [4096,1536]'s bytes in its layout (one wave per row, 3 vectors per lane), "
                "stores held until hold_ticks (10 ns) after each wave's start",
        "bytes": 4 * nb, "buffer_sets_rotated": ns,
        "holds": [{"hold_ticks": h, "us": round(sorted(times[h])[2], 2),
                   "GB/s": round(4 * nb / (sorted(times[h])[2] * 1e-6) / 1e9, 1)} for h in holds]}
    del sets
    torch.cuda.empty_cache()
    return out


def phase_timeline(args, torch, np, W, dev, sp, timer):
    """Per-wave phase stamps of the Llama-405B per-token E4M3 norm
    ([2048, 16384]) from the measurement build libaarms_stamps.so (real-time
    clock, 100 MHz): one launch in the middle of a back-to-back run over
    rotated buffer sets, for the library's default variant (resident rows:
    one wave per row) and for the split rows (16 waves per row) it replaced.
    Reports the launch time with and without the stamps, the per-row (per-
    block) phase times, and over the launch the rows or blocks in flight."""
    import ctypes as C
    from activation_add_rmsnorm_amd import _build
    if not os.path.exists(_build.STAMPS_PATH):
        _build.build()
    L = C.CDLL(_build.STAMPS_PATH)
    vp, i64, f32, i32 = C.c_void_p, C.c_int64, C.c_float, C.c_int
    L.fused_add_rmsnorm_quant_fp8_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
    L.aarms_set_phase_stamps.argtypes = [vp]
    L.aarms_set_phase_stamps.restype = None
    L.aarms_set_phase_stamp_detail.argtypes = [i32]
    L.aarms_set_phase_stamp_detail.restype = None
    L.aarms_pick_variant.argtypes = [i32, i64, i64, i32]
    L.aarms_variant_name.argtypes = [i32, i32]
    L.aarms_variant_name.restype = C.c_char_p
    L.aarms_variant_count.argtypes = [i32]
    wl = W.NORM_FP8_LLAMA405B
    T, H = wl.tokens, wl.hidden
    d = W.norm_inputs(wl)
    to = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    x0, r0, w0 = to(d["x"]), to(d["residual"]), to(d["weight"])
    ns = rotation_sets(norm_bytes(T, H, quant=True))
    sets = [dict(x=x0.clone(), r=r0.clone(), q=torch.empty((T, H), dtype=torch.uint8, device=dev),
                 s=torch.empty((T,), dtype=torch.float32, device=dev), ro=torch.empty_like(r0)) for _ in range(ns)]
    reps = max(20, args.steps // 2)
    pct = lambda v: {"p10": round(float(np.percentile(v, 10)), 2), "median": round(float(np.median(v)), 2),
                     "p90": round(float(np.percentile(v, 90)), 2), "max": round(float(v.max()), 2)}

    def stamped_launch(v, wpr, detail):
        """Plain and stamped launch times, and the stamps [T, wpr, 16] of one
        launch in a back-to-back run."""
        def call(i):
            z = sets[i % ns]
            st = L.fused_add_rmsnorm_quant_fp8_ex(z["q"].data_ptr(), z["s"].data_ptr(), z["ro"].data_ptr(),
                                                   z["x"].data_ptr(), z["r"].data_ptr(), w0.data_ptr(), T, H,
                                                   wl.eps, v, sp)
            if st:
                raise RuntimeError("fused_add_rmsnorm_quant_fp8_ex: %d" % st)
        stamps = torch.zeros(T * wpr * 16, dtype=torch.int64, device=dev)
        L.aarms_set_phase_stamp_detail(1 if detail else 0)
        L.aarms_set_phase_stamps(None)
        timer.warm(call)
        us_plain = timer.region(call, reps) * 1e3
        L.aarms_set_phase_stamps(stamps.data_ptr())
        timer.warm(call)
        us_stamped = timer.region(call, reps) * 1e3
        stamps.zero_()
        torch.cuda.synchronize()
        for i in range(2 * ns):
            call(i)
        torch.cuda.synchronize()
        L.aarms_set_phase_stamps(None)
        L.aarms_set_phase_stamp_detail(0)
        return us_plain, us_stamped, stamps.cpu().numpy().reshape(T, wpr, 16).astype(np.float64)

    def cus_used(a):
        hw, xcc = a[:, 0, 8].astype(np.int64), a[:, 0, 9].astype(np.int64) & 0xF
        cu = ((xcc * 8 + ((hw >> 13) & 7)) * 2 + ((hw >> 12) & 1)) * 16 + ((hw >> 8) & 0xF)
        _, per_cu = np.unique(cu, return_counts=True)
        return int(len(per_cu)), {"min": int(per_cu.min()), "max": int(per_cu.max())}

    def resident(v, vname):
        us_plain, us_stamped, a = stamped_launch(v, 1, False)
        t = (a[:, 0, :] - a[:, 0, 0].min()) * 0.01      # us from the first row's start
        span = float(t[:, 7].max())
        grid = np.linspace(0.0, span, 41)
        ncu, per_cu = cus_used(a)
        return {"variant": vname, "waves_per_row": 1, "launch_us": round(us_plain, 2),
                "launch_us_with_stamps": round(us_stamped, 2), "span_us": round(span, 2),
                "per_row_from_launch_start_us": {
                    "row start": pct(t[:, 0]), "row loads consumed": pct(t[:, 1]),
                    "weight in LDS (block barrier)": pct(t[:, 3]), "row amax computed": pct(t[:, 4]),
                    "last store issued": pct(t[:, 7])},
                "per_row_us": {
                    "start -> row loads consumed": pct(t[:, 1] - t[:, 0]),
                    "loads consumed -> wave sum": pct(t[:, 2] - t[:, 1]),
                    "wave sum -> weight in LDS": pct(t[:, 3] - t[:, 2]),
                    "weight -> row amax computed (amax pass)": pct(t[:, 4] - t[:, 3]),
                    "row amax -> wave maximum": pct(t[:, 5] - t[:, 4]),
                    "wave maximum -> last store issued (quantizing pass)": pct(t[:, 7] - t[:, 5])},
                "grid_us": [round(float(g), 2) for g in grid],
                "rows_loading": [int(((t[:, 0] <= g) & (t[:, 1] > g)).sum()) for g in grid],
                "rows_in_epilogue": [int(((t[:, 1] <= g) & (t[:, 7] > g)).sum()) for g in grid],
                "rows_done": [int((t[:, 7] <= g).sum()) for g in grid],
                "distinct_cus": ncu, "rows_per_cu": per_cu}

    def split(v, vname, wpr):
        us_plain, us_stamped, a = stamped_launch(v, wpr, False)
        t = (a - a[:, :, 0].min()) * 0.01          # us from the first wave's start (slots 8, 9: IDs)
        bstart = t[:, :, 0].min(1)
        span = float(t[:, :, 7].max())
        phases = {
            "last wave's row loads consumed": pct(t[:, :, 1].max(1) - bstart),
            "first wave's row loads consumed": pct(t[:, :, 1].min(1) - bstart),
            "first barrier passed": pct(t[:, :, 3].min(1) - bstart),
            "row amax computed (last wave)": pct(t[:, :, 4].max(1) - bstart),
            "second barrier passed": pct(t[:, :, 6].min(1) - bstart),
            "last store issued (last wave)": pct(t[:, :, 7].max(1) - bstart),
        }
        per_wave = {
            "loads consumed -> wave sum": pct((t[:, :, 2] - t[:, :, 1]).ravel()),
            "first barrier -> row amax computed": pct((t[:, :, 4] - t[:, :, 3]).ravel()),
            "row amax -> wave maximum": pct((t[:, :, 5] - t[:, :, 4]).ravel()),
            "second barrier -> last store issued": pct((t[:, :, 7] - t[:, :, 6]).ravel()),
        }
        # a second pass with the sub-steps of the chain after the first
        # barrier stamped too (more stores and waits in the kernel)
        us_detail, _, ad = stamped_launch(v, wpr, True)
        td = (ad - ad[:, :, 0].min()) * 0.01
        per_wave_detail = {}
        if (ad[:, :, 10:15] > 0).all():
            per_wave_detail = {
                "first barrier -> row sum combined": pct((td[:, :, 10] - td[:, :, 3]).ravel()),
                "row sum -> mean and 1/sqrt": pct((td[:, :, 11] - td[:, :, 10]).ravel()),
                "1/sqrt -> weight in registers": pct((td[:, :, 12] - td[:, :, 11]).ravel()),
                "weight -> row amax computed": pct((td[:, :, 4] - td[:, :, 12]).ravel()),
                "second barrier -> row amax combined": pct((td[:, :, 13] - td[:, :, 6]).ravel()),
                "row amax -> scale and reciprocal": pct((td[:, :, 14] - td[:, :, 13]).ravel()),
                "scale -> last store issued": pct((td[:, :, 7] - td[:, :, 14]).ravel()),
            }
        order = np.argsort(bstart)
        octiles = []
        for g in range(8):
            sl = order[g * T // 8:(g + 1) * T // 8]
            octiles.append({"start_us": round(float(np.median(bstart[sl])), 2),
                            "loads_us": round(float(np.median(t[sl, :, 1].max(1) - bstart[sl])), 2),
                            "barrier1_us": round(float(np.median(t[sl, :, 3].min(1) - bstart[sl])), 2),
                            "barrier2_us": round(float(np.median(t[sl, :, 6].min(1) - bstart[sl])), 2),
                            "end_us": round(float(np.median(t[sl, :, 7].max(1) - bstart[sl])), 2)})
        grid = np.linspace(0.0, span, 41)
        bend = t[:, :, 7].max(1)
        ncu, per_cu = cus_used(a)
        return {"variant": vname, "waves_per_row": wpr, "launch_us": round(us_plain, 2),
                "launch_us_with_stamps": round(us_stamped, 2), "span_us": round(span, 2),
                "per_block_from_block_start_us": phases, "per_wave_us": per_wave, "octiles_by_start": octiles,
                "launch_us_with_detail_stamps": round(us_detail, 2), "per_wave_detail_us": per_wave_detail,
                "grid_us": [round(float(g), 2) for g in grid],
                "blocks_in_flight": [int(((bstart <= g) & (bend > g)).sum()) for g in grid],
                "waves_awaiting_row_loads": [int(((t[:, :, 0] <= g) & (t[:, :, 1] > g)).sum()) for g in grid],
                "distinct_cus": ncu, "blocks_per_cu": per_cu}

    out = {"metric": "per-wave phase timeline, fused_add_rmsnorm_quant_fp8 [2048,16384] (Llama-405B)",
           "buffer_sets_rotated": ns}
    v = L.aarms_pick_variant(0, T, H, 1)
    vname = L.aarms_variant_name(0, v).decode()
    names = {L.aarms_variant_name(0, i).decode(): i for i in range(L.aarms_variant_count(0))}
    if "resident" in vname:
        out["default"] = resident(v, vname)
        progress("phase timeline: split rows")
        out["split_rows"] = split(names["16 waves/row x2 vec"], "16 waves/row x2 vec", 16)
    else:
        wpr = 1 if vname.startswith("wave/row") else int(vname.split()[0])
        out["default"] = split(v, vname, wpr)
    return out


# Supplementary entries and the keys of their traffic lines in profiles/.
TRAFFIC_KEYS = {
    "llama70b_swiglu_fp8_8192x57344": "swiglu_fp8_llama70b",
    "llama405b_norm_fp8_2048x16384": "norm_fp8_llama405b",
    "llama70b_swiglu_nvfp4_8192x57344": "swiglu_nvfp4_llama70b",
}


def supplementary(args, torch, np, A, lib, clib, W, dev, sp, timer, to_dev):
    out = {}
    reps = max(20, args.steps // 2)
    want = (lambda key: re.search(args.configs, key) is not None) if args.configs else (lambda key: True)

    def stream(*a):
        st = clib.aarms_reference_copy(*a, sp)
        if st:
            raise RuntimeError("aarms_reference_copy: %d" % st)

    if want("llama70b_swiglu_fp8_8192x57344"):
        progress("llama70b_swiglu_fp8_8192x57344")
        out.update(config4(torch, A, lib, W, dev, sp, timer, reps, stream))
    if want("llama405b_norm_fp8_2048x16384"):
        progress("llama405b_norm_fp8_2048x16384")
        out.update(config5(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream))
    if want("qwen1.5b_norm_16x1536"):
        progress("qwen1.5b_norm_16x1536")
        out.update(config1(torch, A, lib, W, sp, timer, to_dev, reps))
    if want("qwen1.5b_decode_28layers_graph"):
        progress("qwen1.5b_decode_28layers_graph")
        out["qwen1.5b_decode_28layers_graph"] = decode_graph(torch, np, A, W, dev, to_dev, timer)

    # the rest of the quantisation matrix, at the same shapes
    out.update(quant_matrix(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream, want))

    # one GPU's share of the Llama layers sharded over 8 GPUs
    out.update(shares(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream, want))

    # calibrated HBM traffic per launch, from the committed counter summaries
    # taken on the current kernel sources (else absent)
    src_hash = kernel_sources_hash()
    for key, tkey in TRAFFIC_KEYS.items():
        t = traffic_from_profiles(tkey, src_hash)
        if key in out and t is not None:
            out[key]["traffic_bytes_per_launch"] = t
            out[key]["traffic_over_algorithmic"] = round(t / out[key]["bytes"], 4)

    # start-up autotuning at the workload shapes: the heuristic's variant
    # against the fastest one (graph-replay timings); informational, the
    # figures above use the heuristic
    if not args.no_autotune_report and want("autotune"):
        progress("autotune report")
        out["autotune"] = autotune_report()
    return out


def config4(torch, A, lib, W, dev, sp, timer, reps, stream):
    """Static-FP8 SwiGLU, Llama-70B MLP: [8192, 57344] -> e4m3 [8192, 28672]."""
    out = {}
    wl = W.SWIGLU_FP8_LLAMA70B
    T, N = wl.tokens, wl.inter
    g = torch.Generator(device=dev).manual_seed(0)
    gu = (torch.randn((T, 2 * N), generator=g, device=dev, dtype=torch.float32) * wl.gate_up_std).to(torch.bfloat16)
    n4 = rotation_sets(swiglu_bytes(T, N, quant=True))
    sets = [(gu if i == 0 else gu.clone(), torch.empty((T, N), dtype=torch.uint8, device=dev)) for i in range(n4)]
    scale = torch.tensor([wl.scale], dtype=torch.float32, device=dev)
    ptr = [(o.data_ptr(), a.data_ptr(), scale.data_ptr()) for a, o in sets]

    def call4(i):
        st = lib.swiglu_quant_fp8(*ptr[i % n4], T, N, sp)
        if st:
            raise A.AarmsError(st, "swiglu_quant_fp8")

    def copy4(i):
        o, a, _ = ptr[i % n4]
        stream(o, 8, None, 0, a, a + T * N * 2, T * N // 8)

    timer.warm(call4)
    ms = timer.region(call4, reps)
    timer.warm(copy4)
    ms_c = timer.region(copy4, reps)
    b = swiglu_bytes(T, N, quant=True)
    out["llama70b_swiglu_fp8_8192x57344"] = {"bytes": b, "avg_launch_us": round(ms * 1e3, 2),
                                              "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                                              "pct_of_hbm_peak": round(100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                              **refcopy_entry(ms * 1e3, ms_c * 1e3, b),
                                              "inputs": "torch.randn on device, seed 0, std 2"}
    del sets, gu, ptr
    torch.cuda.empty_cache()
    return out


def config5(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream):
    """Dynamic-FP8 norm, Llama-405B: [2048, 16384]."""
    out = {}
    wl = W.NORM_FP8_LLAMA405B
    T, H = wl.tokens, wl.hidden
    d = W.norm_inputs(wl)
    x0, r0, w0 = to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["weight"])
    b = norm_bytes(T, H, quant=True)
    n_sets = rotation_sets(b)
    sets = []
    for i in range(n_sets):
        s = dict(x=x0.clone(), r=r0.clone(), q=torch.empty((T, H), dtype=torch.uint8, device=dev),
                 s=torch.empty((T,), dtype=torch.float32, device=dev), ro=torch.empty_like(r0))
        s["p"] = (s["q"].data_ptr(), s["s"].data_ptr(), s["ro"].data_ptr(), s["x"].data_ptr(),
                  s["r"].data_ptr(), w0.data_ptr())
        sets.append(s)

    def call5(i):
        st = lib.fused_add_rmsnorm_quant_fp8(*sets[i % n_sets]["p"], T, H, wl.eps, sp)
        if st:
            raise A.AarmsError(st, "fused_add_rmsnorm_quant_fp8")

    def copy5(i):
        s = sets[i % n_sets]
        stream(s["ro"].data_ptr(), 16, s["q"].data_ptr(), 8, s["x"].data_ptr(), s["r"].data_ptr(), T * H // 8)

    timer.warm(call5)
    ms = timer.region(call5, reps)
    timer.warm(copy5)
    ms_c = timer.region(copy5, reps)
    out["llama405b_norm_fp8_2048x16384"] = {"bytes": b, "avg_launch_us": round(ms * 1e3, 2),
                                             "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                                             "pct_of_hbm_peak": round(100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                             **refcopy_entry(ms * 1e3, ms_c * 1e3, b),
                                             "buffer_sets_rotated": n_sets}
    del sets
    torch.cuda.empty_cache()
    return out


def config1(torch, A, lib, W, sp, timer, to_dev, reps):
    """The 16-token norm (launch-bound, microseconds)."""
    out = {}
    wl = W.NORM_DECODE16
    d = W.norm_inputs(wl)
    x, r, w = to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["weight"])
    o, ro = torch.empty_like(x), torch.empty_like(r)
    p = (o.data_ptr(), ro.data_ptr(), x.data_ptr(), r.data_ptr(), w.data_ptr())

    def call1(i):
        lib.fused_add_rmsnorm(*p, wl.tokens, wl.hidden, wl.eps, sp)

    timer.warm(call1, 0.02)
    ms = timer.region(call1, reps)
    out["qwen1.5b_norm_16x1536"] = {"bytes": norm_bytes(16, 1536), "avg_launch_us": round(ms * 1e3, 2)}
    return out


def autotune_report():
    from activation_add_rmsnorm_amd import tuning
    shapes = [("fused_add_rmsnorm", 4096, 1536), ("swiglu", 4096, 8960),
              ("fused_add_rmsnorm", 1, 1536), ("swiglu", 1, 8960),
              ("fused_add_rmsnorm_quant_fp8", 2048, 16384), ("swiglu_quant_fp8", 8192, 28672),
              ("rmsnorm", 4096, 1536), ("rmsnorm_quant_fp8", 2048, 16384),
              ("fused_add_rmsnorm_quant_fp8_static", 2048, 16384), ("swiglu_quant_fp8_dynamic", 8192, 28672),
              ("fused_add_rmsnorm_quant_mxfp4", 2048, 16384), ("swiglu_quant_mxfp4", 8192, 28672),
              ("swiglu_quant_mxfp4", 1, 8960), ("fused_add_rmsnorm_quant_nvfp4", 2048, 16384),
              ("swiglu_quant_nvfp4", 8192, 28672), ("fused_add_rmsnorm_quant_fp8_group", 2048, 16384),
              ("swiglu_quant_fp8_group", 8192, 28672)]
    rows = []
    for form, T, W in shapes:
        r = tuning.tune(form, T, W)
        r["gain_pct"] = round(100 * (r["heuristic_us"] / r["best_us"] - 1), 1)
        rows.append(r)
    tuning.clear()
    return rows


def quant_matrix(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream, want=lambda key: True):
    """rmsnorm (no residual add) at the Qwen prefill shape; the static-scale,
    block-scaled (MXFP4, NVFP4, per-128 E4M3) and no-residual per-token norms
    at the Llama-405B shape; the block-scaled and per-token SwiGLU forms at
    the Llama-70B shape.  Each beside its reference copy, on rotated
    buffer sets."""
    out = {}

    def measure(key, call, refcopy, nbytes, extra=None):
        if not want(key):
            return
        progress(key)
        timer.warm(call)
        ms = timer.region(call, reps)
        timer.warm(refcopy)
        ms_c = timer.region(refcopy, reps)
        e = {"bytes": nbytes, "avg_launch_us": round(ms * 1e3, 2),
             "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
             "pct_of_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
             **refcopy_entry(ms * 1e3, ms_c * 1e3, nbytes)}
        e.update(extra or {})
        out[key] = e

    def check(st, what):
        if st:
            raise A.AarmsError(st, what)

    # rmsnorm bf16 [4096, 1536]
    wl = W.NORM_PREFILL4096
    T, H = wl.tokens, wl.hidden
    d = W.norm_inputs(wl)
    x0, w0 = to_dev(d["x"]), to_dev(d["weight"])
    nb = T * H * 2 * 2 + H * 2
    ns = rotation_sets(nb)
    sets = [(x0.clone(), torch.empty_like(x0)) for _ in range(ns)]
    half = T * H                                      # bytes in half of a bf16 [T, H] tensor
    measure("qwen1.5b_rmsnorm_4096x1536",
            lambda i: check(lib.rmsnorm(sets[i % ns][1].data_ptr(), sets[i % ns][0].data_ptr(),
                                        w0.data_ptr(), T, H, wl.eps, sp), "rmsnorm"),
            lambda i: stream(sets[i % ns][1].data_ptr(), 16, sets[i % ns][1].data_ptr() + half, 16,
                             sets[i % ns][0].data_ptr(), sets[i % ns][0].data_ptr() + half, T * H // 16),
            nb, {"buffer_sets_rotated": ns})
    del sets

    # static-scale FP8 norms and the per-token FP8 norm without the residual, [2048, 16384]
    wl = W.NORM_FP8_LLAMA405B
    T, H = wl.tokens, wl.hidden
    d = W.norm_inputs(wl)
    x0, r0, w0 = to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["weight"])
    scale = torch.tensor([0.02], dtype=torch.float32, device=dev)
    nb = T * H * 7 + H * 2 + 4
    ns = rotation_sets(nb)
    sets = [dict(x=x0.clone(), r=r0.clone(), q=torch.empty((T, H), dtype=torch.uint8, device=dev),
                 ro=torch.empty_like(r0), s=torch.empty((T,), dtype=torch.float32, device=dev))
            for _ in range(ns)]
    P = lambda i, k: sets[i % ns][k].data_ptr()
    measure("llama405b_norm_fp8_static_2048x16384",
            lambda i: check(lib.fused_add_rmsnorm_quant_fp8_static(
                P(i, "q"), P(i, "ro"), P(i, "x"), P(i, "r"), w0.data_ptr(), scale.data_ptr(),
                T, H, wl.eps, sp), "fused_add_rmsnorm_quant_fp8_static"),
            lambda i: stream(P(i, "ro"), 16, P(i, "q"), 8, P(i, "x"), P(i, "r"), T * H // 8),
            nb, {"scale": 0.02, "buffer_sets_rotated": ns})
    mq = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
    ms_ = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    mx_sets = [(mq if i == 0 else torch.empty_like(mq), ms_ if i == 0 else torch.empty_like(ms_)) for i in range(ns)]
    nb = T * H * 6 + T * H // 2 + T * H // 32 + H * 2
    measure("llama405b_norm_mxfp4_2048x16384",
            lambda i: check(lib.fused_add_rmsnorm_quant_mxfp4(
                mx_sets[i % ns][0].data_ptr(), mx_sets[i % ns][1].data_ptr(), P(i, "ro"), P(i, "x"), P(i, "r"),
                w0.data_ptr(), T, H, wl.eps, sp), "fused_add_rmsnorm_quant_mxfp4"),
            lambda i: stream(P(i, "ro"), 16, mx_sets[i % ns][0].data_ptr(), 4, P(i, "x"), P(i, "r"), T * H // 8),
            nb, {"buffer_sets_rotated": ns})
    del mx_sets
    nv_sets = [(torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
                torch.empty((T, H // 16), dtype=torch.uint8, device=dev)) for _ in range(ns)]
    nb = T * H * 6 + T * H // 2 + T * H // 16 + H * 2 + 4
    measure("llama405b_norm_nvfp4_2048x16384",
            lambda i: check(lib.fused_add_rmsnorm_quant_nvfp4(
                nv_sets[i % ns][0].data_ptr(), nv_sets[i % ns][1].data_ptr(), P(i, "ro"), P(i, "x"), P(i, "r"),
                w0.data_ptr(), scale.data_ptr(), T, H, wl.eps, sp), "fused_add_rmsnorm_quant_nvfp4"),
            lambda i: stream(P(i, "ro"), 16, nv_sets[i % ns][0].data_ptr(), 4, P(i, "x"), P(i, "r"), T * H // 8),
            nb, {"tensor_scale": 0.02, "buffer_sets_rotated": ns})
    del nv_sets
    G = A.FP8_GROUP
    gs_sets = [torch.empty((T, H // G), dtype=torch.float32, device=dev) for _ in range(ns)]
    nb = T * H * 7 + T * H // G * 4 + H * 2
    measure("llama405b_norm_fp8_group_2048x16384",
            lambda i: check(lib.fused_add_rmsnorm_quant_fp8_group(
                P(i, "q"), gs_sets[i % ns].data_ptr(), P(i, "ro"), P(i, "x"), P(i, "r"), w0.data_ptr(),
                T, H, wl.eps, sp), "fused_add_rmsnorm_quant_fp8_group"),
            lambda i: stream(P(i, "ro"), 16, P(i, "q"), 8, P(i, "x"), P(i, "r"), T * H // 8),
            nb, {"group": G, "buffer_sets_rotated": ns})
    del gs_sets
    nb = T * H * 3 + H * 2 + T * 4
    measure("llama405b_rmsnorm_fp8_2048x16384",
            lambda i: check(lib.rmsnorm_quant_fp8(P(i, "q"), P(i, "s"), P(i, "x"), w0.data_ptr(),
                                                  T, H, wl.eps, sp), "rmsnorm_quant_fp8"),
            lambda i: stream(P(i, "q"), 16, None, 0, P(i, "x"), P(i, "x") + T * H, T * H // 16),
            nb, {"buffer_sets_rotated": ns})
    del sets, x0, r0

    # per-token FP8 SwiGLU, [8192, 57344] -> e4m3 [8192, 28672]
    wl = W.SWIGLU_FP8_LLAMA70B
    T, N = wl.tokens, wl.inter
    g = torch.Generator(device=dev).manual_seed(0)
    gu = (torch.randn((T, 2 * N), generator=g, device=dev, dtype=torch.float32) * wl.gate_up_std).to(torch.bfloat16)
    nb = T * 2 * N * 2 + T * N + T * 4
    ns = rotation_sets(nb)
    sets = [(gu if i == 0 else gu.clone(), torch.empty((T, N), dtype=torch.uint8, device=dev),
             torch.empty((T,), dtype=torch.float32, device=dev)) for i in range(ns)]
    mx_sets = [(torch.empty((T, N // 2), dtype=torch.uint8, device=dev),
                torch.empty((T, N // 32), dtype=torch.uint8, device=dev)) for _ in range(ns)]
    measure("llama70b_swiglu_mxfp4_8192x57344",
            lambda i: check(lib.swiglu_quant_mxfp4(mx_sets[i % ns][0].data_ptr(), mx_sets[i % ns][1].data_ptr(),
                                                   sets[i % ns][0].data_ptr(), T, N, sp), "swiglu_quant_mxfp4"),
            lambda i: stream(mx_sets[i % ns][0].data_ptr(), 4, None, 0, sets[i % ns][0].data_ptr(),
                             sets[i % ns][0].data_ptr() + T * N * 2, T * N // 8),
            T * 2 * N * 2 + T * N // 2 + T * N // 32,
            {"inputs": "torch.randn on device, seed 0, std 2", "buffer_sets_rotated": ns})
    del mx_sets
    nv_sets = [(torch.empty((T, N // 2), dtype=torch.uint8, device=dev),
                torch.empty((T, N // 16), dtype=torch.uint8, device=dev)) for _ in range(ns)]
    g_nv = torch.tensor([0.05], dtype=torch.float32, device=dev)
    measure("llama70b_swiglu_nvfp4_8192x57344",
            lambda i: check(lib.swiglu_quant_nvfp4(nv_sets[i % ns][0].data_ptr(), nv_sets[i % ns][1].data_ptr(),
                                                   sets[i % ns][0].data_ptr(), g_nv.data_ptr(), T, N, sp),
                            "swiglu_quant_nvfp4"),
            lambda i: stream(nv_sets[i % ns][0].data_ptr(), 4, None, 0, sets[i % ns][0].data_ptr(),
                             sets[i % ns][0].data_ptr() + T * N * 2, T * N // 8),
            T * 2 * N * 2 + T * N // 2 + T * N // 16 + 4,
            {"tensor_scale": 0.05, "inputs": "torch.randn on device, seed 0, std 2", "buffer_sets_rotated": ns})
    del nv_sets
    G = A.FP8_GROUP
    gs_sets = [torch.empty((T, N // G), dtype=torch.float32, device=dev) for _ in range(ns)]
    measure("llama70b_swiglu_fp8_group_8192x57344",
            lambda i: check(lib.swiglu_quant_fp8_group(sets[i % ns][1].data_ptr(), gs_sets[i % ns].data_ptr(),
                                                       sets[i % ns][0].data_ptr(), T, N, sp),
                            "swiglu_quant_fp8_group"),
            lambda i: stream(sets[i % ns][1].data_ptr(), 8, None, 0, sets[i % ns][0].data_ptr(),
                             sets[i % ns][0].data_ptr() + T * N * 2, T * N // 8),
            T * 2 * N * 2 + T * N + T * N // G * 4,
            {"group": G, "inputs": "torch.randn on device, seed 0, std 2", "buffer_sets_rotated": ns})
    del gs_sets
    measure("llama70b_swiglu_fp8_dynamic_8192x57344",
            lambda i: check(lib.swiglu_quant_fp8_dynamic(sets[i % ns][1].data_ptr(), sets[i % ns][2].data_ptr(),
                                                         sets[i % ns][0].data_ptr(), T, N, sp),
                            "swiglu_quant_fp8_dynamic"),
            lambda i: stream(sets[i % ns][1].data_ptr(), 8, None, 0, sets[i % ns][0].data_ptr(),
                             sets[i % ns][0].data_ptr() + T * N * 2, T * N // 8),
            nb, {"inputs": "torch.randn on device, seed 0, std 2", "buffer_sets_rotated": ns})
    del sets, gu
    torch.cuda.empty_cache()
    return out


def shares(torch, A, lib, W, dev, sp, timer, to_dev, reps, stream, want=lambda key: True):
    """The kernels on one GPU's share of the sharded layers: the 405B FP8
    norm on T/8 = 256 rows (sequence parallel), the 70B static-FP8 SwiGLU on
    N/8 = 3,584 columns of gate and of up (tensor parallel).  Each beside its
    reference copy, on rotated buffer sets."""
    out = {}

    def entry(ms, ms_c, nbytes, extra):
        return {"bytes": nbytes, "avg_launch_us": round(ms * 1e3, 2),
                "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "pct_of_hbm_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                **refcopy_entry(ms * 1e3, ms_c * 1e3, nbytes), **extra}

    def check(st, what):
        if st:
            raise A.AarmsError(st, what)

    wl = W.NORM_FP8_LLAMA405B_SP8
    if want(wl.name):
        _share_norm(out, wl, torch, A, lib, dev, sp, timer, to_dev, reps, stream, entry, check, W)
    wl = W.SWIGLU_FP8_LLAMA70B_TP8
    if want(wl.name):
        _share_swiglu(out, wl, torch, A, lib, dev, sp, timer, reps, stream, entry, check)
    torch.cuda.empty_cache()
    return out


def _share_norm(out, wl, torch, A, lib, dev, sp, timer, to_dev, reps, stream, entry, check, W):
    T, H = wl.tokens, wl.hidden
    d = W.norm_inputs(wl)
    x0, r0, w0 = to_dev(d["x"]), to_dev(d["residual"]), to_dev(d["weight"])
    nb = norm_bytes(T, H, quant=True)
    ns = rotation_sets(nb)
    sets = [dict(x=x0.clone(), r=r0.clone(), q=torch.empty((T, H), dtype=torch.uint8, device=dev),
                 s=torch.empty((T,), dtype=torch.float32, device=dev), ro=torch.empty_like(r0))
            for _ in range(ns)]
    P = lambda i, k: sets[i % ns][k].data_ptr()
    call = lambda i: check(lib.fused_add_rmsnorm_quant_fp8(P(i, "q"), P(i, "s"), P(i, "ro"), P(i, "x"), P(i, "r"),
                                                           w0.data_ptr(), T, H, wl.eps, sp),
                           "fused_add_rmsnorm_quant_fp8")
    refcopy = lambda i: stream(P(i, "ro"), 16, P(i, "q"), 8, P(i, "x"), P(i, "r"), T * H // 8)
    timer.warm(call)
    ms = timer.region(call, reps)
    timer.warm(refcopy)
    ms_c = timer.region(refcopy, reps)
    out[wl.name] = entry(ms, ms_c, nb, {"buffer_sets_rotated": ns})
    del sets, x0, r0


def _share_swiglu(out, wl, torch, A, lib, dev, sp, timer, reps, stream, entry, check):
    T, N = wl.tokens, wl.inter
    g = torch.Generator(device=dev).manual_seed(0)
    gu = (torch.randn((T, 2 * N), generator=g, device=dev, dtype=torch.float32) * wl.gate_up_std).to(torch.bfloat16)
    nb = swiglu_bytes(T, N, quant=True)
    ns = rotation_sets(nb)
    sets = [(gu if i == 0 else gu.clone(), torch.empty((T, N), dtype=torch.uint8, device=dev)) for i in range(ns)]
    scale = torch.tensor([wl.scale], dtype=torch.float32, device=dev)
    call = lambda i: check(lib.swiglu_quant_fp8(sets[i % ns][1].data_ptr(), sets[i % ns][0].data_ptr(),
                                                scale.data_ptr(), T, N, sp), "swiglu_quant_fp8")
    refcopy = lambda i: stream(sets[i % ns][1].data_ptr(), 8, None, 0, sets[i % ns][0].data_ptr(),
                            sets[i % ns][0].data_ptr() + T * N * 2, T * N // 8)
    timer.warm(call)
    ms = timer.region(call, reps)
    timer.warm(refcopy)
    ms_c = timer.region(refcopy, reps)
    out[wl.name] = entry(ms, ms_c, nb, {"inputs": "torch.randn on device, seed 0, std 2", "buffer_sets_rotated": ns})
    del sets, gu


def decode_graph(torch, np, A, W, dev, to_dev, timer):
    wl = W.DECODE_GRAPH
    res = {}
    for T in wl.tokens:
        H, N, L = wl.hidden, wl.inter, wl.layers
        host = [W.decode_layer_inputs(wl, T, l) for l in range(L)]
        r = to_dev(W.decode_residual(wl, T))
        bufs = []
        for h in host:
            bufs.append(dict(x1=to_dev(h["x1"]), x2=to_dev(h["x2"]), w1=to_dev(h["w1"]), w2=to_dev(h["w2"]),
                             gu=to_dev(h["gate_up"]), o1=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
                             o2=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
                             y=torch.empty((T, N), dtype=torch.bfloat16, device=dev)))

        def chain():
            for b in bufs:
                A.fused_add_rmsnorm(b["x1"], r, b["w1"], wl.eps, out=b["o1"], residual_out=r)
                A.fused_add_rmsnorm(b["x2"], r, b["w2"], wl.eps, out=b["o2"], residual_out=r)
                A.swiglu(b["gu"], out=b["y"])

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            chain()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            chain()
        timer.warm(lambda i: g.replay(), 0.05)
        reps = 50
        ms_graph = timer.region(lambda i: g.replay(), reps)
        ms_eager = timer.region(lambda i: chain(), 10)
        byts = L * (2 * norm_bytes(T, H) + swiglu_bytes(T, N))
        res["T=%d" % T] = {"us_per_replay": round(ms_graph * 1e3, 1),
                           "us_per_node": round(ms_graph * 1e3 / (3 * L), 2),
                           "us_eager_python": round(ms_eager * 1e3, 1),
                           "bytes": byts, "GB/s": round(byts / (ms_graph * 1e-3) / 1e9, 1)}
        del g, bufs
        torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo where there is one."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(np, W, nd, gd, step_bytes, seconds):
    """The oracle as it stands, on the headline workload, repeated for a
    bounded time on all of the host's cores, then on one core over a row
    sample of the same workload."""
    import oracle
    wl = W.NORM_PREFILL4096
    oracle.fused_add_rmsnorm(nd["x"][:8], nd["residual"][:8], nd["weight"], wl.eps)  # warm
    cores = oracle.num_threads()

    def timed(rows, budget):
        x, r, gu = nd["x"][:rows], nd["residual"][:rows], gd["gate_up"][:rows]
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.fused_add_rmsnorm(x, r, nd["weight"], wl.eps)
            oracle.swiglu(gu)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or el > 3 * budget:
                return reps, el

    T = nd["x"].shape[0]
    reps, el = timed(T, seconds)
    out = {"value": round(step_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": cores,
           "kind": "oracle", "sample": "%d full passes of the headline workload (norm [4096,1536] + "
                                       "swiglu [4096,17920]) in %.1f s" % (reps, el),
           "ms_per_step": round(el / reps * 1e3, 1), "cpu_model": cpu_model()}
    # one core, on the first 256 rows of the same tensors (the bytes scale with rows)
    rows = 256
    oracle.set_threads(1)
    try:
        reps1, el1 = timed(rows, max(1.0, seconds / 5))
    finally:
        oracle.set_threads(cores)
    out["single_core"] = {"value": round(step_bytes * rows / T * reps1 / el1 / 1e9, 3), "unit": "GB/s",
                          "cores": 1, "sample": "%d passes over the first %d rows of the headline workload "
                                                "in %.1f s" % (reps1, rows, el1),
                          "ms_per_step": round(el1 / reps1 * T / rows * 1e3, 1)}
    return out


if __name__ == "__main__":
    main()
