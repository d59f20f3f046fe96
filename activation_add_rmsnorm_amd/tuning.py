"""Startup variant autotuning, cached per (op form, row width, token bucket).

The plain entry points choose a kernel variant with a fixed heuristic
(include/aarms.h, aarms_pick_variant).  No variant is fastest for every
shape; the first page's tuning study finds near-ties among versions flipping
from run to run and only large gaps stable ("TensorRT-LLM: Compiling
Inference Engines Ahead of Time", section "Auto-tuning, measured"), and its
runtime tunes at start-up per shape bucket with a cache saved to a file and
reloaded (section "Leaving the engine behind").  ``tune()`` times every
variant that fits one (form, tokens, width) on this device, on rotated
buffer sets so that each launch reads HBM, and installs the fastest in this
process's table only when it beats the heuristic's choice by more than
``margin``, so a near-tie never flips the choice.  The Python entry points
of this package consult the table when called with ``variant=-1``; the C
library itself stays stateless.  Tokens are bucketed to the next power of
two.  ``save()`` / ``load()`` keep the table in a JSON file tied to the
library build and device, so a stale table is ignored rather than applied.

Each variant's launches are captured once into a HIP graph and the graph is
replayed between HIP events, so host launch overhead does not hide the
kernels' own differences at small shapes.  The graphs are replayed for a
while before any is timed (clocks settle under load), then timed
interleaved, and the median of the rounds is kept.  This module allocates
its own buffers and synchronizes: call it at start-up, not inside a
captured graph.
"""

from __future__ import annotations

import hashlib
import json
import math
import os
import time

import torch

import activation_add_rmsnorm_amd as A

MALL_BYTES = 256e6          # MI355X last-level cache; rotation covers three times this

# form -> (variant table op, the quant argument of aarms_pick_variant: the
# output format; norms: 0 bf16, 1 E4M3 per token, 2 E4M3 per tensor,
# 3 MXFP4, 4 NVFP4, 5 E4M3 per group; swiglu: 0 bf16, 1 E4M3, 2 MXFP4,
# 3 NVFP4, 4 E4M3 per group)
FORMS = {
    "fused_add_rmsnorm": (A.OP_NORM, 0),
    "fused_add_rmsnorm_quant_fp8": (A.OP_NORM, 1),
    "fused_add_rmsnorm_quant_fp8_static": (A.OP_NORM, 2),
    "rmsnorm": (A.OP_RMSNORM, 0),
    "rmsnorm_quant_fp8": (A.OP_RMSNORM, 1),
    "rmsnorm_quant_fp8_static": (A.OP_RMSNORM, 2),
    "fused_add_rmsnorm_quant_mxfp4": (A.OP_NORM, 3),
    "rmsnorm_quant_mxfp4": (A.OP_RMSNORM, 3),
    "swiglu": (A.OP_SWIGLU, 0),
    "swiglu_quant_fp8": (A.OP_SWIGLU, 1),
    "swiglu_quant_fp8_dynamic": (A.OP_SWIGLU_DYNAMIC, True),
    "swiglu_quant_mxfp4": (A.OP_SWIGLU, 2),
    "fused_add_rmsnorm_quant_nvfp4": (A.OP_NORM, 4),
    "rmsnorm_quant_nvfp4": (A.OP_RMSNORM, 4),
    "swiglu_quant_nvfp4": (A.OP_SWIGLU, 3),
    "fused_add_rmsnorm_quant_fp8_group": (A.OP_NORM, 5),
    "rmsnorm_quant_fp8_group": (A.OP_RMSNORM, 5),
    "swiglu_quant_fp8_group": (A.OP_SWIGLU, 4),
}


def bucket(tokens: int) -> int:
    """The power of two at or above tokens (1 for 0 or 1)."""
    t = max(1, int(tokens))
    return 1 << (t - 1).bit_length()


def _key(form: str, tokens: int, width: int):
    if form not in FORMS:
        raise ValueError("unknown form %r" % form)
    return (form, int(width), bucket(tokens))


def set_variant(form: str, tokens: int, width: int, variant: int) -> None:
    A._TUNED[_key(form, tokens, width)] = int(variant)


def variant_for(form: str, tokens: int, width: int) -> int:
    """The tuned variant for this call, or -1 (the library's heuristic)."""
    return A._TUNED.get(_key(form, tokens, width), -1)


def clear() -> None:
    A._TUNED.clear()


def variants_fitting(form: str, width: int):
    op, _ = FORMS[form]
    return [v for v in range(A.variant_count(op)) if A.variant_fits(op, v, width)]


def _buffers(form: str, tokens: int, width: int, device):
    """One set of inputs and outputs for a launch of `form`, and its bytes."""
    T, W = int(tokens), int(width)
    bf = dict(dtype=torch.bfloat16, device=device)
    f8 = dict(dtype=torch.uint8, device=device)
    if form.startswith("swiglu"):
        b = dict(gu=(torch.randn((T, 2 * W), device=device) * 2).to(torch.bfloat16))
        if "fp4" in form:
            blk = 32 if "mxfp4" in form else 16
            b["y"] = torch.empty((T, W // 2), **f8)
            b["s"] = torch.empty((T, W // blk), **f8)
            nbytes = T * W * 4 + T * W // 2 + T * W // blk
        else:
            b["y"] = torch.empty((T, W), **(f8 if "fp8" in form else bf))
            b["s"] = torch.empty((T, W // A.FP8_GROUP) if "group" in form else (T,), dtype=torch.float32,
                                 device=device)
            nbytes = T * W * 4 + T * W * (1 if "fp8" in form else 2)
    else:
        b = dict(x=torch.randn((T, W), device=device).to(torch.bfloat16),
                 r=torch.randn((T, W), device=device).to(torch.bfloat16))
        if "fp4" in form:
            blk = 32 if "mxfp4" in form else 16
            b["o"] = torch.empty((T, W // 2), **f8)
            b["s"] = torch.empty((T, W // blk), **f8)
            out_bytes = T * W // 2 + T * W // blk
        else:
            b["o"] = torch.empty((T, W), **(f8 if "fp8" in form else bf))
            b["s"] = torch.empty((T, W // A.FP8_GROUP) if "group" in form else (T,), dtype=torch.float32,
                                 device=device)
            out_bytes = T * W * (1 if "fp8" in form else 2)
        b["ro"] = torch.empty((T, W), **bf)
        nbytes = T * W * (2 if form.startswith("rmsnorm") else 6) + out_bytes
    return b, nbytes


def _launcher(form: str, b: dict, w, scale, variant: int):
    if form == "fused_add_rmsnorm":
        return lambda: A.fused_add_rmsnorm(b["x"], b["r"], w, 1e-6, out=b["o"], residual_out=b["ro"], variant=variant)
    if form == "fused_add_rmsnorm_quant_fp8":
        return lambda: A.fused_add_rmsnorm_quant_fp8(b["x"], b["r"], w, 1e-6, out=b["o"], scale_out=b["s"],
                                                     residual_out=b["ro"], variant=variant)
    if form == "fused_add_rmsnorm_quant_fp8_static":
        return lambda: A.fused_add_rmsnorm_quant_fp8_static(b["x"], b["r"], w, scale, 1e-6, out=b["o"],
                                                            residual_out=b["ro"], variant=variant)
    if form == "rmsnorm":
        return lambda: A.rmsnorm(b["x"], w, 1e-6, out=b["o"], variant=variant)
    if form == "rmsnorm_quant_fp8":
        return lambda: A.rmsnorm_quant_fp8(b["x"], w, 1e-6, out=b["o"], scale_out=b["s"], variant=variant)
    if form == "rmsnorm_quant_fp8_static":
        return lambda: A.rmsnorm_quant_fp8_static(b["x"], w, scale, 1e-6, out=b["o"], variant=variant)
    if form == "fused_add_rmsnorm_quant_mxfp4":
        return lambda: A.fused_add_rmsnorm_quant_mxfp4(b["x"], b["r"], w, 1e-6, out=b["o"], scale_out=b["s"],
                                                       residual_out=b["ro"], variant=variant)
    if form == "rmsnorm_quant_mxfp4":
        return lambda: A.rmsnorm_quant_mxfp4(b["x"], w, 1e-6, out=b["o"], scale_out=b["s"], variant=variant)
    if form == "swiglu":
        return lambda: A.swiglu(b["gu"], out=b["y"], variant=variant)
    if form == "swiglu_quant_fp8":
        return lambda: A.swiglu_quant_fp8(b["gu"], scale, out=b["y"], variant=variant)
    if form == "fused_add_rmsnorm_quant_nvfp4":
        return lambda: A.fused_add_rmsnorm_quant_nvfp4(b["x"], b["r"], w, scale, 1e-6, out=b["o"], scale_out=b["s"],
                                                       residual_out=b["ro"], variant=variant)
    if form == "rmsnorm_quant_nvfp4":
        return lambda: A.rmsnorm_quant_nvfp4(b["x"], w, scale, 1e-6, out=b["o"], scale_out=b["s"], variant=variant)
    if form == "swiglu_quant_nvfp4":
        return lambda: A.swiglu_quant_nvfp4(b["gu"], scale, out=b["y"], scale_out=b["s"], variant=variant)
    if form == "swiglu_quant_mxfp4":
        return lambda: A.swiglu_quant_mxfp4(b["gu"], out=b["y"], scale_out=b["s"], variant=variant)
    if form == "fused_add_rmsnorm_quant_fp8_group":
        return lambda: A.fused_add_rmsnorm_quant_fp8_group(b["x"], b["r"], w, 1e-6, out=b["o"], scale_out=b["s"],
                                                           residual_out=b["ro"], variant=variant)
    if form == "rmsnorm_quant_fp8_group":
        return lambda: A.rmsnorm_quant_fp8_group(b["x"], w, 1e-6, out=b["o"], scale_out=b["s"], variant=variant)
    if form == "swiglu_quant_fp8_group":
        return lambda: A.swiglu_quant_fp8_group(b["gu"], out=b["y"], scale_out=b["s"], variant=variant)
    if form == "swiglu_quant_fp8_dynamic":
        return lambda: A.swiglu_quant_fp8_dynamic(b["gu"], out=b["y"], scale_out=b["s"], variant=variant)
    raise ValueError(form)


def sweep(form: str, tokens: int, width: int, rounds: int = 5, device=None, max_sets: int = 64,
          warm_s: float = 0.1, only=None):
    """Mean time per launch in microseconds of every fitting variant (the
    median of `rounds` timed regions each), on rotated buffer sets.

    All variants are captured first; their graphs are then replayed in turn
    for about `warm_s` seconds, so that the clocks have settled under load
    (after the host has left the device idle they take some tens of
    milliseconds, and a kernel with more arithmetic per byte is slowed more
    until they have), and finally timed interleaved, round by round.
    `only`: time these variant ids instead of every fitting one."""
    device = torch.device(device or "cuda")
    first, nbytes = _buffers(form, tokens, width, device)
    sets = [first]
    n_sets = min(max_sets, max(2, math.ceil(3 * MALL_BYTES / max(nbytes, 1))))
    for _ in range(n_sets - 1):
        sets.append({k: (v.clone() if k in ("x", "r", "gu") else torch.empty_like(v)) for k, v in first.items()})
    W = int(width)
    w = (1 + 0.1 * torch.randn((W,), device=device)).to(torch.bfloat16) if not form.startswith("swiglu") else None
    scale = torch.tensor([0.05], dtype=torch.float32, device=device)
    # about 2 ms of work per replay, at least 8 launches (a whole number of
    # passes over the buffer sets)
    est_us = max(nbytes / 5e3, 2.0)
    reps = max(8, min(512, int(2000 / est_us)))
    reps = max(n_sets, reps - reps % n_sets)
    graphs = {}
    for v in (variants_fitting(form, W) if only is None else only):
        calls = [_launcher(form, s, w, scale, v) for s in sets]
        side = torch.cuda.Stream(device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            for c in calls:
                c()
        torch.cuda.current_stream(device).wait_stream(side)
        torch.cuda.synchronize(device)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                calls[i % len(calls)]()
        graphs[v] = g
    torch.cuda.synchronize(device)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize(device)
    samples = {v: [] for v in graphs}
    for _ in range(rounds):
        marks = []
        for v, g in graphs.items():
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            e.record()
            marks.append((v, a, e))
        torch.cuda.synchronize(device)
        for v, a, e in marks:
            samples[v].append(a.elapsed_time(e) * 1e3 / reps)
    del graphs
    return {v: sorted(x)[len(x) // 2] for v, x in samples.items()}


def tune(form: str, tokens: int, width: int, margin: float = 0.03, rounds: int = 5, device=None):
    """Time every fitting variant and install the fastest for (form, bucket of
    tokens, width) if it beats the heuristic's pick by more than `margin`,
    in the sweep and again in a second timing of the two alone.
    Returns a report: the heuristic's pick and time, the best and its time,
    and the variant installed (-1: the heuristic stays)."""
    op, quant = FORMS[form]
    # time at the bucket's token count, the shape every call in it shares best
    T = bucket(tokens)
    times = sweep(form, T, width, rounds=rounds, device=device)
    pick = A.pick_variant(op, T, width, quant)
    best = min(times, key=times.get)
    chosen = best if (pick not in times or times[best] < times[pick] * (1 - margin)) else -1
    if chosen >= 0 and pick in times:
        # a second, independent timing of the two must confirm the gain
        again = sweep(form, T, width, rounds=2 * rounds + 1, device=device, only=[pick, best])
        if not again[best] < again[pick] * (1 - margin):
            chosen = -1
    if chosen >= 0:
        set_variant(form, T, width, chosen)
    name = lambda v: A.variant_name(op, v) if v >= 0 else None
    return {"form": form, "tokens_bucket": T, "width": int(width),
            "heuristic": name(pick), "heuristic_us": round(times.get(pick, float("nan")), 3),
            "best": name(best), "best_us": round(times[best], 3), "installed": name(chosen)}


def _identity() -> dict:
    """The library build and the device kind a table belongs to."""
    h = hashlib.sha256(open(A.lib_path(), "rb").read()).hexdigest()[:16]
    if torch.cuda.is_available():
        dev = torch.cuda.get_device_properties(torch.cuda.current_device())
        name, arch = dev.name, getattr(dev, "gcnArchName", "")
    else:
        name, arch = "none", ""
    return {"library_sha256": h, "device": name, "arch": arch}


def save(path: str) -> None:
    entries = [{"form": f, "width": w, "tokens_bucket": t, "variant": v} for (f, w, t), v in A._TUNED.items()]
    with open(path, "w") as fh:
        json.dump({"identity": _identity(), "entries": entries}, fh, indent=1)


def load(path: str) -> int:
    """Install the entries of a saved table made by this library build on this
    kind of device; returns the number installed (0 for a stale file)."""
    if not os.path.exists(path):
        return 0
    with open(path) as fh:
        data = json.load(fh)
    if data.get("identity") != _identity():
        return 0
    n = 0
    for e in data.get("entries", []):
        if e["form"] in FORMS:
            A._TUNED[(e["form"], int(e["width"]), int(e["tokens_bucket"]))] = int(e["variant"])
            n += 1
    return n
