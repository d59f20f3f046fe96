"""Build libaarms.so (the library) and libaarms_refcopy.so (plain streaming
copies that bench.py times beside the library kernels) in-tree with hipcc for
gfx950.

Flags:
  -ffp-contract=off    no implicit fused multiply-add: every fma in the kernels
                       is written out, so the rounding points are the ones in
                       the source;
  -fhip-fp32-correctly-rounded-divide-sqrt
                       IEEE binary32 division (per-row scale and reciprocal);
  -Xclang -target-feature -Xclang -packed-fp32-ops
                       no packed binary32 instructions;
  -fvisibility=hidden  only the functions include/aarms.h declares are exported.
No fast-math, no denormal flushing (binary32 and binary64 denormals are kept).
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libaarms.so")
REFCOPY_PATH = os.path.join(PKG, "libaarms_refcopy.so")
# Measurement build: the library with phase stamps in the norm kernels
# (-DAARMS_PHASE_STAMPS, bench.py --phase-timeline); never loaded by the
# package itself.
STAMPS_PATH = os.path.join(PKG, "libaarms_stamps.so")
ARCH = os.environ.get("AARMS_OFFLOAD_ARCH", "gfx950")

HIP_SOURCES = ["norm.hip", "norm_resident.hip", "swiglu.hip"]
HOST_SOURCES = ["capi.cpp"]
REFCOPY_SOURCES = ["refcopy.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
          "-ffp-contract=off", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _run(jobs, verbose):
    procs = []
    for cmd in jobs:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = False
    for cmd, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is expected
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l
                         and "is not a recognized feature" not in l)
        if text.strip():
            print(text, file=sys.stderr)
        if pr.returncode != 0:
            failed = True
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed")


def _link(hipcc, objs, path):
    tmp = path + ".tmp%d" % os.getpid()
    subprocess.run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs], check=True)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source, link libaarms.so, libaarms_refcopy.so and
    libaarms_stamps.so; returns the path of libaarms.so."""
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)

    def obj(src):
        return os.path.join(objdir, src + ".o")

    def sobj(src):
        return os.path.join(objdir, src + ".stamps.o")

    stamps = ["-DAARMS_PHASE_STAMPS"]
    jobs = [[hipcc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, s), "-o", obj(s)]
            for s in HIP_SOURCES + REFCOPY_SOURCES]
    jobs += [[hipcc, *COMMON, "-c", os.path.join(CSRC, s), "-o", obj(s)] for s in HOST_SOURCES]
    jobs += [[hipcc, *COMMON, *DEVICE, *stamps, "-c", os.path.join(CSRC, s), "-o", sobj(s)]
             for s in ("norm.hip", "norm_resident.hip")]
    jobs += [[hipcc, *COMMON, *stamps, "-c", os.path.join(CSRC, "capi.cpp"), "-o", sobj("capi.cpp")]]
    _run(jobs, verbose)
    _link(hipcc, [obj(s) for s in HIP_SOURCES + HOST_SOURCES], LIB_PATH)
    _link(hipcc, [obj(s) for s in REFCOPY_SOURCES], REFCOPY_PATH)
    _link(hipcc, [sobj("norm.hip"), sobj("norm_resident.hip"), obj("swiglu.hip"), sobj("capi.cpp")],
          STAMPS_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
