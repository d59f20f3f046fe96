"""The C ABI without a GPU: libaarms.so loads, exports every function that
include/aarms.h declares, and rejects bad arguments before any HIP call.

Only error paths are called here (validation returns before anything is
enqueued), plus the variant tables; no kernel is launched.  Pointer values
are plain integers that are never dereferenced.
"""

from __future__ import annotations

import ctypes as C
import os
import re
import subprocess

import activation_add_rmsnorm_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aarms.h")

OK, NULLP, SHAPE, UNSUP, MISAL, ALIAS, EPS, HIP, VARIANT = range(9)
MAX_HIDDEN = 65536


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_four_ops():
    fns = declared_functions()
    for name in ["fused_add_rmsnorm", "swiglu", "swiglu_quant_fp8", "fused_add_rmsnorm_quant_fp8",
                 "aarms_status_string", "rmsnorm", "rmsnorm_quant_fp8", "rmsnorm_quant_fp8_static",
                 "fused_add_rmsnorm_quant_fp8_static", "swiglu_quant_fp8_dynamic"]:
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = A.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_library_exports_only_declared_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", A.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == set(declared_functions()), exported ^ set(declared_functions())


def test_library_imports_no_allocation_or_synchronization():
    """The header's promise that the library never allocates, frees or
    synchronizes, checked on the built library: everything it imports is
    kernel registration, the current device and its attributes, the
    occupancy calculator, the launch, and the C++ runtime's start-up hooks.
    No hipMalloc, hipFree, *Synchronize, blocking copy or host heap."""
    out = subprocess.run(["nm", "-D", "--undefined-only", A.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = {l.split()[-1].split("@")[0] for l in out.splitlines() if l.strip()}
    # a sanitizer build (tests/test_host_sanitizers.py) also imports its runtime's hooks
    imported = {n for n in imported if not n.startswith(("__asan_", "__ubsan_", "__sanitizer_", "__lsan_"))}
    allowed = {"__hipRegisterFatBinary", "__hipUnregisterFatBinary", "__hipRegisterFunction",
               "__hipPopCallConfiguration", "__hipPushCallConfiguration", "hipLaunchKernel", "hipGetDevice",
               "hipDeviceGetAttribute", "hipOccupancyMaxActiveBlocksPerMultiprocessor",
               "__cxa_atexit", "__cxa_finalize", "__deregister_frame_info", "__register_frame_info",
               "__gmon_start__", "_ITM_deregisterTMCloneTable", "_ITM_registerTMCloneTable",
               # other compilers' builds of the host code (the sanitizer test's): guarded
               # initialization of function-local statics, the stack protector
               "__cxa_guard_acquire", "__cxa_guard_release", "__cxa_guard_abort", "__stack_chk_fail"}
    assert imported <= allowed, sorted(imported - allowed)


def test_status_strings():
    lib = A.load()
    for s in range(9):
        txt = lib.aarms_status_string(s)
        assert txt and txt != b"unknown status"
    assert lib.aarms_status_string(99) == b"unknown status"


# ----------------------------------------------------------------- norms

P = 0x10000  # an aligned fake device address; buffers are placed far apart
BIG = 1 << 32


def norm(lib, out=P, res_out=P + BIG, x=P + 2 * BIG, res=P + 3 * BIG, w=P + 4 * BIG,
         T=4, H=1536, eps=1e-6):
    return lib.fused_add_rmsnorm(out, res_out, x, res, w, T, H, eps, None)


def normq(lib, out=P, scale=P + BIG, res_out=P + 2 * BIG, x=P + 3 * BIG, res=P + 4 * BIG,
          w=P + 5 * BIG, T=4, H=1536, eps=1e-6):
    return lib.fused_add_rmsnorm_quant_fp8(out, scale, res_out, x, res, w, T, H, eps, None)


def test_norm_shape_errors():
    lib = A.load()
    assert norm(lib, T=-1) == SHAPE
    assert norm(lib, H=0) == SHAPE
    assert norm(lib, H=-8) == SHAPE
    assert norm(lib, H=12) == SHAPE
    assert norm(lib, H=MAX_HIDDEN + 8) == UNSUP
    assert norm(lib, T=1 << 31, H=8) == UNSUP
    assert norm(lib, T=1 << 30, H=4096) == UNSUP          # beyond 2^40 elements
    assert normq(lib, H=20) == SHAPE


def test_norm_zero_tokens_is_a_noop():
    lib = A.load()
    assert norm(lib, T=0, out=0, res_out=0, x=0, res=0, w=0) == OK
    assert normq(lib, T=0, out=0, scale=0, res_out=0, x=0, res=0, w=0) == OK
    assert norm(lib, T=0, H=12) == SHAPE                    # the shape is still checked


def test_norm_eps_errors():
    lib = A.load()
    for eps in [-1e-6, float("nan"), float("inf"), -float("inf")]:
        assert norm(lib, eps=eps) == EPS
        assert normq(lib, eps=eps) == EPS


def test_norm_null_and_alignment():
    lib = A.load()
    for k in ["out", "res_out", "x", "res", "w"]:
        assert norm(lib, **{k: 0}) == NULLP
        assert norm(lib, **{k: P + 8 + {"out": 0, "res_out": 1, "x": 2, "res": 3, "w": 4}[k] * BIG}) == MISAL
    assert normq(lib, scale=0) == NULLP
    assert normq(lib, scale=P + BIG + 2) == MISAL


def test_norm_aliasing_rules():
    """Calls that pass the aliasing rules are stopped before launch by a
    variant too narrow for the row (checked last)."""
    lib = A.load()
    T, H = 4, 1536
    n = T * H * 2
    x = P + 2 * BIG
    res = P + 3 * BIG
    w = P + 4 * BIG
    narrow = 0                                  # one wave, one vector per lane: 512 wide
    assert A.variant_name(A.OP_NORM, narrow) == "wave/row x1 vec"
    # exact in-place pairs are allowed
    assert lib.fused_add_rmsnorm_ex(x, res, x, res, w, T, H, 1e-6, narrow, None) == VARIANT
    # out overlapping residual_out
    assert norm(lib, out=P, res_out=P + 16) == ALIAS
    # out == residual (not an allowed pair)
    assert norm(lib, out=res) == ALIAS
    # partial overlap with x
    assert norm(lib, out=x + 16) == ALIAS
    # residual_out overlapping the weight
    assert norm(lib, res_out=w - 16) == ALIAS
    # adjacent, non-overlapping buffers are fine
    assert lib.fused_add_rmsnorm_ex(P, P + n, P + 2 * n, P + 3 * n, P + 4 * n, T, H, 1e-6,
                                    narrow, None) == VARIANT
    # quant: out_fp8 may not alias x; residual_out may alias residual
    assert normq(lib, out=P + 3 * BIG) == ALIAS
    assert lib.fused_add_rmsnorm_quant_fp8_ex(P, P + BIG, P + 4 * BIG, P + 3 * BIG, P + 4 * BIG,
                                              P + 5 * BIG, T, H, 1e-6, narrow, None) == VARIANT
    # scale_out overlapping out
    assert normq(lib, scale=P + 64) == ALIAS


def test_norm_variant_checks():
    lib = A.load()
    n = A.variant_count(A.OP_NORM)
    assert n >= 10
    args = (P, P + BIG, P + 2 * BIG, P + 3 * BIG, P + 4 * BIG)
    assert lib.fused_add_rmsnorm_ex(*args, 4, 1536, 1e-6, n, None) == VARIANT
    assert lib.fused_add_rmsnorm_ex(*args, 4, 1536, 1e-6, -2, None) == VARIANT
    # a variant too narrow for the row is refused before launch
    narrow = [i for i in range(n) if "wave/row x1" in A.variant_name(A.OP_NORM, i)][0]
    assert lib.fused_add_rmsnorm_ex(*args, 4, 1536, 1e-6, narrow, None) == VARIANT
    assert A.variant_name(A.OP_NORM, n) is None
    # the resident-row variants: rows up to 16,384 wide, multiples of 512
    resident = [i for i in range(n) if "resident" in A.variant_name(A.OP_NORM, i)]
    assert len(resident) == 2
    for i in resident:
        for H, ok in ((512, True), (1536, True), (16384, True), (12800, True), (1544, False),
                      (16376, False), (16896, False), (8, False)):
            assert A.variant_fits(A.OP_NORM, i, H) == ok, (i, H)
            assert A.variant_fits(A.OP_RMSNORM, i, H) == ok, (i, H)
        assert lib.fused_add_rmsnorm_ex(*args, 4, 1544, 1e-6, i, None) == VARIANT
        assert lib.fused_add_rmsnorm_quant_fp8_ex(P, P + BIG, P + 2 * BIG, P + 3 * BIG, P + 4 * BIG,
                                                  P + 5 * BIG, 4, 16376, 1e-6, i, None) == VARIANT
    # the fit query agrees with the capacity rule everywhere else
    for i in range(n):
        name = A.variant_name(A.OP_NORM, i)
        w = 1 if name.startswith("wave/row") else int(name.split()[0])
        cap = w * 64 * int(name.split("x")[-1].split()[0]) * 8
        for H in (8, 1536, 4096, 4104, 16384, 65536):
            expect = cap >= H and ("resident" not in name or H % 512 == 0)
            assert A.variant_fits(A.OP_NORM, i, H) == expect, (name, H)
    assert not A.variant_fits(A.OP_NORM, n, 1536) and not A.variant_fits(A.OP_NORM, -1, 1536)
    assert not A.variant_fits(7, 0, 1536)
    for v in range(A.variant_count(A.OP_SWIGLU)):
        assert A.variant_fits(A.OP_SWIGLU, v, 8960) and not A.variant_fits(A.OP_SWIGLU, v, 12)


# ----------------------------------------------------------------- the other norm forms

def rms(lib, out=P, x=P + BIG, w=P + 2 * BIG, T=4, H=1536, eps=1e-6, variant=-1):
    return lib.rmsnorm_ex(out, x, w, T, H, eps, variant, None)


def rmsq(lib, out=P, scale=P + BIG, x=P + 2 * BIG, w=P + 3 * BIG, T=4, H=1536, eps=1e-6, variant=-1):
    return lib.rmsnorm_quant_fp8_ex(out, scale, x, w, T, H, eps, variant, None)


def rmss(lib, out=P, x=P + BIG, w=P + 2 * BIG, scale=P + 3 * BIG, T=4, H=1536, eps=1e-6, variant=-1):
    return lib.rmsnorm_quant_fp8_static_ex(out, x, w, scale, T, H, eps, variant, None)


def norms(lib, out=P, res_out=P + BIG, x=P + 2 * BIG, res=P + 3 * BIG, w=P + 4 * BIG,
          scale=P + 5 * BIG, T=4, H=1536, eps=1e-6, variant=-1):
    return lib.fused_add_rmsnorm_quant_fp8_static_ex(out, res_out, x, res, w, scale, T, H, eps,
                                                     variant, None)


def test_other_norm_forms_errors():
    lib = A.load()
    narrow = 0
    for f in (rms, rmsq, rmss, norms):
        assert f(lib, T=-1) == SHAPE
        assert f(lib, H=12) == SHAPE
        assert f(lib, H=MAX_HIDDEN + 8) == UNSUP
        assert f(lib, eps=float("nan")) == EPS
        assert f(lib, out=0) == NULLP
        assert f(lib, out=P + 8) == MISAL
        assert f(lib, variant=A.variant_count(A.OP_NORM)) == VARIANT
        assert f(lib, variant=narrow) == VARIANT                # too narrow, stops before launch
    assert rms(lib, T=0, out=0, x=0, w=0) == OK
    assert rmsq(lib, T=0, out=0, scale=0, x=0, w=0) == OK
    assert rmss(lib, T=0, out=0, x=0, w=0, scale=0) == OK
    assert norms(lib, T=0, out=0, res_out=0, x=0, res=0, w=0, scale=0) == OK
    assert rmsq(lib, scale=0) == NULLP
    assert rmsq(lib, scale=P + BIG + 2) == MISAL
    assert rmss(lib, scale=0) == NULLP
    assert rmss(lib, scale=P + 3 * BIG + 1) == MISAL
    assert norms(lib, scale=0) == NULLP
    assert norms(lib, res=0) == NULLP
    assert norms(lib, res_out=P + BIG + 8) == MISAL


def test_other_norm_forms_aliasing():
    lib = A.load()
    x, w = P + BIG, P + 2 * BIG
    # rmsnorm: out == x in place is allowed (stopped by the narrow variant)
    assert rms(lib, out=x, variant=0) == VARIANT
    assert rms(lib, out=x + 16) == ALIAS
    assert rms(lib, out=w - 16) == ALIAS
    # FP8 forms: no in-place output
    assert rmsq(lib, out=P + 2 * BIG) == ALIAS
    assert rmss(lib, out=P + BIG) == ALIAS
    assert rmsq(lib, scale=P + 64) == ALIAS                   # scale_out inside out
    assert rmss(lib, scale=P + 64) == ALIAS                   # scale inside out
    # static fused form: residual_out == residual allowed, out == x not
    assert norms(lib, res_out=P + 3 * BIG, variant=0) == VARIANT
    assert norms(lib, out=P + 2 * BIG) == ALIAS
    assert norms(lib, res_out=P + 5 * BIG) == ALIAS           # residual_out over the scale


# ----------------------------------------------------------------- swiglu

def sw(lib, out=P, gu=P + BIG, T=4, N=8960):
    return lib.swiglu(out, gu, T, N, None)


def swq(lib, out=P, gu=P + BIG, scale=P + 2 * BIG, T=4, N=8960):
    return lib.swiglu_quant_fp8(out, gu, scale, T, N, None)


def test_swiglu_errors():
    lib = A.load()
    assert sw(lib, T=-1) == SHAPE
    assert sw(lib, N=0) == SHAPE
    assert sw(lib, N=12) == SHAPE
    assert sw(lib, T=1 << 20, N=1 << 20) == UNSUP
    assert sw(lib, T=0, out=0, gu=0) == OK
    assert sw(lib, out=0) == NULLP
    assert sw(lib, gu=0) == NULLP
    assert sw(lib, out=P + 2) == MISAL
    assert sw(lib, gu=P + BIG + 8) == MISAL
    assert sw(lib, out=P + BIG) == ALIAS                       # in place is not allowed
    assert sw(lib, out=P + BIG + 4 * 8960 * 4 - 16) == ALIAS   # tail overlap
    assert swq(lib, scale=0) == NULLP
    assert swq(lib, scale=P + 2 * BIG + 2) == MISAL
    assert swq(lib, scale=P + 4) == ALIAS                      # scale inside out
    assert swq(lib, T=0, out=0, gu=0, scale=0) == OK
    n = A.variant_count(A.OP_SWIGLU)
    assert lib.swiglu_ex(P, P + BIG, 4, 8960, n, None) == VARIANT
    # more rows than the launch grids can index (within the element limit)
    assert sw(lib, T=(1 << 31), N=8) == UNSUP
    assert sw(lib, T=(1 << 31) - 1, N=8, out=0) == NULLP       # the limit itself passes the shape checks
    assert swq(lib, T=1 << 31, N=8) == UNSUP


def swd(lib, out=P, scale=P + BIG, gu=P + 2 * BIG, T=4, N=8960, variant=-1):
    return lib.swiglu_quant_fp8_dynamic_ex(out, scale, gu, T, N, variant, None)


def test_swiglu_dynamic_errors():
    lib = A.load()
    assert swd(lib, T=1 << 31, N=8) == UNSUP
    assert swd(lib, T=-1) == SHAPE
    assert swd(lib, N=12) == SHAPE
    assert swd(lib, N=65536 + 8) == UNSUP                   # row kept in registers
    assert swd(lib, T=0, out=0, scale=0, gu=0) == OK
    for k in ("out", "scale", "gu"):
        assert swd(lib, **{k: 0}) == NULLP
    assert swd(lib, out=P + 8) == MISAL
    assert swd(lib, scale=P + BIG + 2) == MISAL
    assert swd(lib, out=P + 2 * BIG) == ALIAS
    assert swd(lib, scale=P + 64) == ALIAS
    n = A.variant_count(A.OP_SWIGLU_DYNAMIC)
    assert swd(lib, variant=n) == VARIANT
    assert swd(lib, variant=0) == VARIANT                   # one wave, one job: 512 wide
    assert A.pick_variant(A.OP_SWIGLU_DYNAMIC, 16, 65544) == -1
    for N in (8, 2048, 8960, 28672, 65536):
        v = A.pick_variant(A.OP_SWIGLU_DYNAMIC, 16, N)
        name = A.variant_name(A.OP_SWIGLU_DYNAMIC, v)
        waves = 1 if name.startswith("wave/row") else int(name.split()[0])
        jobs = int(name.split("x")[-1].split()[0])
        assert waves * 64 * jobs * 8 >= N


def test_swiglu_width_limit():
    lib = A.load()
    P = 1 << 40
    assert lib.swiglu(P, P + (1 << 45), 1, (1 << 33) + 8, None) == UNSUP
    assert lib.swiglu_quant_fp8(P, P + (1 << 45), P - 64, 1, (1 << 33) + 8, None) == UNSUP


def test_pick_variant_ranges():
    for H in [8, 512, 520, 1536, 4096, 4104, 8192, 16384, 32768, 65536]:
        v = A.pick_variant(A.OP_NORM, 16, H)
        assert v >= 0, H
    assert A.pick_variant(A.OP_NORM, 16, MAX_HIDDEN + 8) == -1
    assert A.pick_variant(A.OP_SWIGLU, 16, 8960) >= 0
    assert A.pick_variant(A.OP_SWIGLU, 16, 12) == -1
    assert A.pick_variant(A.OP_SWIGLU, 16, 8960, 5) == -1          # unknown output format
    assert A.pick_variant(A.OP_SWIGLU, 16, 8960, -1) == -1
    name = lambda T, N, f: A.variant_name(A.OP_SWIGLU, A.pick_variant(A.OP_SWIGLU, T, N, f))
    # decode sizes: half jobs; E4M3 from ~4 M outputs: the flat grid, two
    # jobs per lane on rows of 256 jobs; NVFP4: two jobs only from ~32 M
    # outputs on rows of whole 512-job blocks; per-group E4M3: one job
    assert name(16, 8960, 0) == name(16, 8960, 3) == "1 half job/lane"
    assert name(4096, 8960, 0) == name(4096, 8960, 2) == "1 job/lane"
    assert name(4096, 8960, 1) == name(2048, 5632, 1) == name(8192, 3584, 1) == "1 job/lane, flat rows"
    assert name(8192, 28672, 1) == "1 job/lane, flat rows" and name(8192, 2048, 1) == "2 jobs/lane"
    assert name(256, 8960, 1) == "1 job/lane, flat rows"                      # E4M3 from ~2 M outputs
    # rows ending in a partial block over an even number of blocks (whose
    # partial blocks would land on half the XCDs): the flat grid
    for f in (0, 2, 3, 4):
        for N in (7168, 11008, 18944):
            assert name(4096, N, f) == "1 job/lane, flat rows", (N, f)
        for N in (5632, 8960, 9728, 13824, 14336):                            # odd counts, whole blocks
            assert name(4096, N, f) == "1 job/lane", (N, f)
    # rows of 257-511 jobs: the flat grid in every format (past the decode sizes)
    for f in range(5):
        assert name(8192, 3584, f) == name(4096, 2056, f) == "1 job/lane, flat rows", f
    assert name(8192, 2048, 0) == name(8192, 4096, 0) == "1 job/lane"
    assert name(4096, 8960, 3) == "1 job/lane"
    assert name(8192, 28672, 3) == "2 jobs/lane" and name(512, 28672, 3) == "1 job/lane"
    assert name(4096, 8960, 4) == name(8192, 14336, 4) == "1 job/lane"
    assert name(8192, 28672, 4) == name(512, 28672, 4) == "1 job/lane"
    assert name(16, 8960, 4) == "1 half job/lane"
    # norms: the output format decides only for per-token E4M3 with the residual
    # on rows wider than 8,192 up to 1,024 tokens (two row reductions: fewer waves)
    nname = lambda op, T, H, f: A.variant_name(op, A.pick_variant(op, T, H, f))
    for f in (0, 2, 3, 4, 5):
        assert nname(A.OP_NORM, 256, 16384, f) == "16 waves/row x2 vec"
    assert nname(A.OP_NORM, 256, 16384, 1) == "8 waves/row x4 vec"
    assert nname(A.OP_NORM, 1, 12288, 1) == "8 waves/row x4 vec"
    assert nname(A.OP_NORM, 768, 16384, 1) == "8 waves/row x4 vec"
    # 12,289-16,384 wide (multiples of 512): resident rows at 0.8-1 and 1.75-2
    # four-row blocks per CU (256 CUs without a device) for per-token and
    # per-tensor E4M3 with the add and bf16 with and without it; the split
    # rows between the bands, around them and for the other forms
    W6, W10 = "wave/row x32 vec, resident, 6-slice window", "wave/row x32 vec, resident, 10-slice window"
    for f in (0, 1, 2):
        for T in (832, 1000, 1024):
            assert nname(A.OP_NORM, T, 16384, f) == W6, (T, f)
        for T in (1792, 2040, 2048):                     # 2,048 per-token: the 405B workload
            assert nname(A.OP_NORM, T, 16384, f) == W10, (T, f)
        assert nname(A.OP_NORM, 2048, 12800, f) == W10
        assert nname(A.OP_NORM, 1536, 16384, f) == nname(A.OP_NORM, 2049, 16384, f) == "16 waves/row x2 vec"
        assert nname(A.OP_NORM, 2048, 16376, f) == "16 waves/row x2 vec"
    assert nname(A.OP_RMSNORM, 1024, 16384, 0) == nname(A.OP_RMSNORM, 2048, 16384, 0) == W6
    assert nname(A.OP_RMSNORM, 1536, 16384, 0) == "8 waves/row x4 vec, pipelined 2 blocks/CU"
    for f in (3, 4, 5):
        assert "resident" not in nname(A.OP_NORM, 2048, 16384, f), f
    for f in (1, 2, 3, 4, 5):
        assert "resident" not in nname(A.OP_RMSNORM, 2048, 16384, f), f
    assert nname(A.OP_NORM, 256, 8192, 1) == nname(A.OP_NORM, 768, 8192, 0) == "8 waves/row x2 vec"
    # with the add, the resident rows (6-slice window) also on rows of
    # 10,240-12,288 in both bands, and for bf16 on 6,144-9,728 in the second
    for f in (0, 1, 2):
        for H in (10240, 12288):
            for T in (832, 1024, 1792, 2048):
                assert nname(A.OP_NORM, T, H, f) == W6, (T, H, f)
            assert "resident" not in nname(A.OP_NORM, 1536, H, f)
            assert "resident" not in nname(A.OP_NORM, 2049, H, f)
            assert "resident" not in nname(A.OP_RMSNORM, 1024, H, f)          # not without the add
        assert "resident" not in nname(A.OP_NORM, 2048, 10248, f)             # a multiple of 512 only
    for H in (6144, 8192, 9728):
        assert nname(A.OP_NORM, 1792, H, 0) == nname(A.OP_NORM, 2048, H, 0) == W6, H
        assert "resident" not in nname(A.OP_NORM, 1024, H, 0), H
        for f in (1, 2):
            assert "resident" not in nname(A.OP_NORM, 2048, H, f), (H, f)
    assert "resident" not in nname(A.OP_NORM, 2048, 5632, 0)
    # narrow rows: four waves per row for small batches; with the residual
    # add (every form but per-token E4M3) up to 2,047 tokens on rows of
    # 1,025-1,536 and 1,799 on rows of 1,537-2,048, up to 1,535 tokens of
    # 1,024 or less (bf16), else up to 1,023
    for f in (0, 2, 3, 4, 5):
        for H, last in ((1536, 2047), (1544, 1799), (2048, 1799)):
            assert nname(A.OP_NORM, last, H, f) == "4 waves/row x1 vec", (H, f)
            assert nname(A.OP_NORM, last + 1, H, f).startswith("wave/row"), (H, f)
        assert nname(A.OP_NORM, 1023, 1024, f) == "4 waves/row x1 vec", f
    assert nname(A.OP_NORM, 1535, 1024, 0) == "4 waves/row x1 vec"
    assert nname(A.OP_NORM, 1536, 1024, 0) == "wave/row x2 vec"
    for f in (2, 3, 4, 5):
        assert nname(A.OP_NORM, 1024, 1024, f) == "wave/row x2 vec", f
    assert nname(A.OP_NORM, 4096, 1536, 0) == "wave/row x3 vec"                # the headline norm
    assert nname(A.OP_NORM, 1023, 1536, 1) == "4 waves/row x1 vec"
    assert nname(A.OP_NORM, 1024, 1536, 1) == "wave/row x3 vec"
    for f in (0, 1, 2, 3, 4, 5):
        assert nname(A.OP_RMSNORM, 1023, 1536, f) == "4 waves/row x1 vec", f
        assert nname(A.OP_RMSNORM, 1024, 1536, f) == "wave/row x3 vec", f
    assert nname(A.OP_RMSNORM, 256, 16384, 1) == nname(A.OP_RMSNORM, 256, 16384, 0)
    for f in (-1, 6):
        assert A.pick_variant(A.OP_NORM, 16, 1536, f) == -1            # unknown output format
    for op in (A.OP_NORM, A.OP_RMSNORM, A.OP_SWIGLU, A.OP_SWIGLU_DYNAMIC):
        assert A.pick_variant(op, -1, 1536) == -1                      # what the entry points reject
        assert A.pick_variant(op, 16, 1540) == -1
        assert A.pick_variant(op, 0, 1536) >= 0                        # zero tokens is a valid call
    # bf16 with the residual, 4,097-8,192 wide: 4 waves x 4 at 1,024-1,280
    # tokens and 2 waves x 8 at 1,281-1,536 (one generation of blocks)
    for T, H in ((1024, 5120), (1024, 8192), (1280, 6144), (1024, 4104)):
        assert nname(A.OP_NORM, T, H, 0) == "4 waves/row x4 vec", (T, H)
    for T, H in ((1281, 5120), (1536, 6144), (1536, 8192)):
        assert nname(A.OP_NORM, T, H, 0) == "2 waves/row x8 vec", (T, H)
    for T, H in ((768, 5120), (1023, 8192), (1537, 8192), (1024, 12800)):
        assert nname(A.OP_NORM, T, H, 0) == nname(A.OP_NORM, T, H, 2), (T, H)   # the general rule
    assert nname(A.OP_NORM, 1024, 8192, 1) == "8 waves/row x2 vec"      # not the quantised forms
    assert "pipelined" not in nname(A.OP_RMSNORM, 1024, 8192, 0)        # nor without the add at 8,192
    # without the add, rows of 2,049-4,096: one wave per row in bf16 at
    # 1,792-3,072 tokens and at 4,096 (256 CUs), per-token E4M3 on rows up
    # to 3,072 at 1,792-4,096 tokens
    for T in (1792, 3072, 4096):
        assert nname(A.OP_RMSNORM, T, 3072, 0) == nname(A.OP_RMSNORM, T, 3072, 1) == "wave/row x6 vec", T
        assert nname(A.OP_RMSNORM, T, 4096, 0) == "wave/row x8 vec", T
    for T in (1791, 3073, 4095, 4097):
        assert nname(A.OP_RMSNORM, T, 4096, 0) == "2 waves/row x4 vec", T
    assert nname(A.OP_RMSNORM, 2048, 4096, 1) == nname(A.OP_RMSNORM, 4097, 3072, 1) == "2 waves/row x4 vec"
    # small batches with the add on rows of 2,049-8,192: one vector per lane
    # (bf16 up to 512 tokens; per-token E4M3 up to 64 tokens of 2,049-4,096)
    for T in (1, 64, 512):
        assert nname(A.OP_NORM, T, 3072, 0) == nname(A.OP_NORM, T, 4096, 0) == "8 waves/row x1 vec", T
        assert nname(A.OP_NORM, T, 5120, 0) == nname(A.OP_NORM, T, 8192, 0) == "16 waves/row x1 vec", T
    assert nname(A.OP_NORM, 513, 4096, 0) == "4 waves/row x2 vec"
    assert nname(A.OP_NORM, 513, 8192, 0) == "8 waves/row x2 vec"
    assert nname(A.OP_NORM, 64, 4096, 1) == "8 waves/row x1 vec"
    assert nname(A.OP_NORM, 65, 4096, 1) == nname(A.OP_NORM, 64, 4096, 2) == "4 waves/row x2 vec"
    assert nname(A.OP_NORM, 1, 8192, 1) == "8 waves/row x2 vec"
    # with the add on rows of 2,049-4,096 at 1,792-2,048 tokens (one
    # generation of two waves per SIMD): one wave per row, bf16 and per-token E4M3
    for f in (0, 1):
        assert nname(A.OP_NORM, 1792, 3072, f) == nname(A.OP_NORM, 2048, 3072, f) == "wave/row x6 vec", f
        assert nname(A.OP_NORM, 2048, 4096, f) == nname(A.OP_NORM, 1800, 2560, f).replace("x6", "x8"), f
        assert nname(A.OP_NORM, 1787, 4096, f) == "4 waves/row x2 vec", f     # 447 blocks: below the band
    assert nname(A.OP_NORM, 2048, 4096, 2) == "4 waves/row x2 vec"      # not the per-tensor form
    # bf16 with the add on rows of 2,049-4,096: 2 waves x 4 at 2,049-2,560
    # tokens (one wave per row just below, 4 waves x 2 above)
    for H in (2560, 3584, 4096):
        assert nname(A.OP_NORM, 2049, H, 0) == nname(A.OP_NORM, 2560, H, 0) == "2 waves/row x4 vec", H
        assert nname(A.OP_NORM, 2048, H, 0).startswith("wave/row"), H
        assert nname(A.OP_NORM, 2561, H, 0) == ("wave/row x8 vec" if H <= 3072 else "4 waves/row x2 vec"), H
    # and one wave per row on rows of 2,049-3,072: 8 vectors at 2,561-3,072
    # tokens, the fewest that fit at 4,096
    for T in (2561, 3072):
        assert nname(A.OP_NORM, T, 3072, 0) == nname(A.OP_NORM, T, 2560, 0) == "wave/row x8 vec", T
    assert nname(A.OP_NORM, 4096, 3072, 0) == nname(A.OP_NORM, 4096, 2560, 0) == "wave/row x6 vec"
    for T in (3073, 4095, 4097):
        assert nname(A.OP_NORM, T, 3072, 0) == "4 waves/row x2 vec", T
    assert nname(A.OP_NORM, 3072, 3072, 1) == "4 waves/row x2 vec"
    for f in (1, 2):
        assert nname(A.OP_NORM, 2304, 4096, f) == "4 waves/row x2 vec", f    # E4M3 forms: unchanged
    # without the add: 4 waves x 2 below 1,024 tokens up to 4,096 wide; the
    # pipelined 8 x 4 for bf16 at 8,193-16,384 wide from 512 to 2,048 tokens
    assert nname(A.OP_RMSNORM, 512, 4096, 0) == nname(A.OP_RMSNORM, 1, 4096, 1) == "4 waves/row x2 vec"
    assert nname(A.OP_RMSNORM, 1024, 4096, 0) == "2 waves/row x4 vec"
    assert nname(A.OP_RMSNORM, 768, 16384, 0) == "8 waves/row x4 vec, pipelined 2 blocks/CU"
    assert nname(A.OP_RMSNORM, 1024, 16384, 1) == nname(A.OP_RMSNORM, 4096, 16384, 0) == "8 waves/row x4 vec"
    # per-token SwiGLU: several waves per row take at most 3 jobs before 4
    rq = lambda N: A.variant_name(A.OP_SWIGLU_DYNAMIC, A.pick_variant(A.OP_SWIGLU_DYNAMIC, 64, N))
    assert rq(2048) == "wave/row x4 jobs" and rq(5632) == "8 waves/row x2 jobs"
    assert rq(8960) == "8 waves/row x3 jobs" and rq(14336) == "16 waves/row x2 jobs"
    assert rq(28672) == "16 waves/row x4 jobs"


def test_reference_copy_library_rejects_bad_arguments():
    # the plain streaming copies bench.py times beside each op: only their
    # argument checks run here (they return before any HIP call)
    from activation_add_rmsnorm_amd import _build
    if not os.path.exists(_build.REFCOPY_PATH):
        _build.build()
    lib = C.CDLL(_build.REFCOPY_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
    f = lib.aarms_reference_copy
    f.argtypes = [vp, i32, vp, i32, vp, vp, i64, vp]
    P = 1 << 40
    assert f(P, 16, P + (1 << 30), 16, P + (2 << 30), P + (3 << 30), 0, None) == 0   # empty: no launch
    assert f(P, 16, P, 16, P, P, -1, None) == -1
    assert f(P, 12, None, 0, P, P, 8, None) == -1                                     # bad width
    assert f(P, 16, None, 8, P, P, 8, None) == -1                                     # out1 missing
    assert f(P, 16, None, 0, P + 8, P, 8, None) == -1                                 # misaligned
    assert f(P, 16, None, 0, P, P, (2**31) * 256, None) == -1                         # grid too large
    d = lib.aarms_copy_design
    d.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, i64, vp]
    assert d(0, 1, 1, 0, P, None, P + (1 << 30), P + (2 << 30), 0, None) == 0        # empty: no launch
    assert d(7, 1, 1, 0, P, P, P, P, 8, None) == -1                                   # bad kind
    assert d(-1, 1, 1, 0, P, P, P, P, 8, None) == -1
    assert d(3, 1, 1, 0, P, None, P, None, 8, None) == -1                             # read-only: in1 missing
    assert d(5, 1, 1, 0, P, None, None, None, 8, None) == -1                          # copy: in0 missing
    assert d(6, 1, 1, 0, P + 4, None, P, P, 8, None) == -1                            # 8-byte out0 misaligned
    assert d(0, 3, 1, 0, P, None, P, P, 8, None) == -1                                # bad vectors per lane
    assert d(1, 1, 1, 0, P, None, P, P, 8, None) == -1                                # out1 missing
    assert d(2, 1, 1, 0, P, P + 4, P, P, 8, None) == -1                               # out1 misaligned
    assert d(0, 1, 1, -1, P, None, P, P, 8, None) == -1                               # negative grid


def test_binding_types_every_declared_function():
    # ctypes converts a Python float only through a declared argument type:
    # every function of the header must have one in the binding
    lib = A.load()
    missing = [n for n in declared_functions() if getattr(lib, n).argtypes is None]
    assert not missing, missing


def test_mxfp4_norm_errors():
    lib = A.load()

    def mx(out=P, s=P + BIG + 1, ro=P + 2 * BIG, x=P + 3 * BIG, r=P + 4 * BIG, w=P + 5 * BIG, T=4, H=1536,
           variant=-1):
        return lib.fused_add_rmsnorm_quant_mxfp4_ex(out, s, ro, x, r, w, T, H, 1e-6, variant, None)

    assert mx(H=1544) == SHAPE                          # a multiple of 8 but not of 32
    assert mx(s=0) == NULLP
    assert mx(out=P + 4) == MISAL
    assert mx(variant=0) == VARIANT                     # unaligned E8M0 scale bytes are fine
    assert mx(s=P + 100) == ALIAS                       # scales inside the codes
    assert mx(ro=P + 3 * BIG) == ALIAS                  # residual_out over x
    assert mx(ro=P + 4 * BIG, variant=0) == VARIANT     # residual_out == residual in place
    assert mx(T=0, out=0, s=0, ro=0, x=0, r=0, w=0) == OK
    assert lib.rmsnorm_quant_mxfp4_ex(P, P + BIG, P + 2 * BIG, P + 3 * BIG, 4, 40, 1e-6, -1, None) == SHAPE
    assert lib.rmsnorm_quant_mxfp4_ex(P, P + BIG, P + 2 * BIG, P + 3 * BIG, 4, 1536, 1e-6, 0, None) == VARIANT


def test_swiglu_mxfp4_errors():
    lib = A.load()

    def smx(out=P, s=P + BIG + 3, gu=P + 2 * BIG, T=4, N=8960, variant=-1):
        return lib.swiglu_quant_mxfp4_ex(out, s, gu, T, N, variant, None)

    assert smx(N=8968) == SHAPE                          # a multiple of 8, not of 32
    assert smx(s=0) == NULLP
    assert smx(out=P + 8) == MISAL
    assert smx(s=P + 64) == ALIAS                        # scales inside the codes
    assert smx(out=P + 2 * BIG) == ALIAS
    assert smx(variant=A.variant_count(A.OP_SWIGLU)) == VARIANT
    assert smx(T=0, out=0, s=0, gu=0) == OK


def test_nvfp4_errors():
    lib = A.load()
    G = P + 6 * BIG                                   # the tensor scale

    def nv(out=P, s=P + BIG + 1, ro=P + 2 * BIG, x=P + 3 * BIG, r=P + 4 * BIG, w=P + 5 * BIG, g=G,
           T=4, H=1536, variant=-1):
        return lib.fused_add_rmsnorm_quant_nvfp4_ex(out, s, ro, x, r, w, g, T, H, 1e-6, variant, None)

    assert nv(H=1544) == SHAPE                          # a multiple of 8 but not of 16
    assert nv(g=0) == NULLP
    assert nv(s=0) == NULLP
    assert nv(g=G + 2) == MISAL
    assert nv(out=P + 8) == MISAL
    assert nv(s=P + 64) == ALIAS
    assert nv(g=P + 8) == ALIAS                         # tensor scale inside the codes
    assert nv(variant=0) == VARIANT
    assert nv(T=0, out=0, s=0, ro=0, x=0, r=0, w=0, g=0) == OK
    assert lib.rmsnorm_quant_nvfp4_ex(P, P + BIG, P + 2 * BIG, P + 3 * BIG, G, 4, 40, 1e-6, -1, None) == SHAPE
    assert lib.swiglu_quant_nvfp4_ex(P, P + BIG, P + 2 * BIG, G, 4, 8968, -1, None) == SHAPE
    assert lib.swiglu_quant_nvfp4_ex(P, P + BIG, P + 2 * BIG, 0, 4, 8960, -1, None) == NULLP
    assert lib.swiglu_quant_nvfp4_ex(P, P + 64, P + 2 * BIG, G, 4, 8960, -1, None) == ALIAS


def test_fp8_group_errors():
    lib = A.load()

    def fg(out=P, s=P + BIG, ro=P + 2 * BIG, x=P + 3 * BIG, r=P + 4 * BIG, w=P + 5 * BIG, T=4, H=1536,
           variant=-1):
        return lib.fused_add_rmsnorm_quant_fp8_group_ex(out, s, ro, x, r, w, T, H, 1e-6, variant, None)

    def rg(out=P, s=P + BIG, x=P + 3 * BIG, w=P + 5 * BIG, T=4, H=1536, variant=-1):
        return lib.rmsnorm_quant_fp8_group_ex(out, s, x, w, T, H, 1e-6, variant, None)

    def sg(out=P, s=P + BIG, gu=P + 2 * BIG, T=4, N=8960, variant=-1):
        return lib.swiglu_quant_fp8_group_ex(out, s, gu, T, N, variant, None)

    assert A.FP8_GROUP == 128
    for f in (fg, rg):
        assert f(H=1544) == SHAPE                       # a multiple of 8, not of 128
        assert f(H=MAX_HIDDEN + 128) == UNSUP
        assert f(s=0) == NULLP
        assert f(s=P + BIG + 2) == MISAL                # fp32 scales
        assert f(out=P + 8) == MISAL
        assert f(s=P + 64) == ALIAS                     # scales inside the codes
        assert f(out=P + 3 * BIG) == ALIAS              # no in-place output
        assert f(variant=0) == VARIANT                  # too narrow, stops before launch
        assert f(variant=A.variant_count(A.OP_NORM)) == VARIANT
        assert f(T=1 << 31) == UNSUP
    assert fg(ro=P + 4 * BIG, variant=0) == VARIANT     # residual_out == residual in place
    assert fg(ro=P + 3 * BIG) == ALIAS                  # residual_out over x
    assert fg(ro=P + BIG + 16) == ALIAS                 # residual_out over the scales
    assert fg(T=0, out=0, s=0, ro=0, x=0, r=0, w=0) == OK
    assert rg(T=0, out=0, s=0, x=0, w=0) == OK
    assert sg(N=8968) == SHAPE
    assert sg(s=0) == NULLP
    assert sg(s=P + BIG + 1) == MISAL
    assert sg(out=P + 8) == MISAL
    assert sg(s=P + 64) == ALIAS
    assert sg(out=P + 2 * BIG) == ALIAS
    assert sg(variant=A.variant_count(A.OP_SWIGLU)) == VARIANT
    assert sg(T=1 << 31, N=128) == UNSUP
    assert sg(T=0, out=0, s=0, gu=0) == OK
    assert lib.swiglu_quant_fp8_group(P, P + BIG, P + 2 * BIG, 4, 8968, None) == SHAPE
    assert lib.fused_add_rmsnorm_quant_fp8_group(P, P + BIG, P + 2 * BIG, P + 3 * BIG, P + 4 * BIG,
                                                 P + 5 * BIG, 4, 1544, 1e-6, None) == SHAPE
    assert lib.rmsnorm_quant_fp8_group(P, P + BIG, P + 3 * BIG, P + 5 * BIG, 4, 1544, 1e-6, None) == SHAPE


def test_missing_library_fails_loudly(tmp_path):
    """A copy of the package without libaarms.so and without the sources to
    build it: load() must raise (there is no CPU fallback)."""
    import shutil
    import sys
    pkg = tmp_path / "activation_add_rmsnorm_amd"
    pkg.mkdir()
    src = os.path.join(ROOT, "activation_add_rmsnorm_amd")
    for f in ("__init__.py", "_build.py", "tuning.py"):
        shutil.copy(os.path.join(src, f), pkg / f)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import activation_add_rmsnorm_amd as A\n"
            "assert A.lib_path().startswith(%r)\n"
            "try:\n    A.load()\nexcept Exception as e:\n    print('raised', type(e).__name__)\n"
            "else:\n    print('loaded')\n") % (str(tmp_path), str(tmp_path))
    env = {k: v for k, v in os.environ.items() if k != "AARMS_LIB"}   # the copy's own path
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=str(tmp_path),
                       env=env)
    assert "raised" in r.stdout, r.stdout + r.stderr
    assert not os.path.exists(pkg / "libaarms.so")
