"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C oracle (oracle/aarms_oracle.c) and the C entry points of the library
(activation_add_rmsnorm_amd/csrc/capi.cpp: argument validation, variant
choice) are rebuilt with -fsanitize=address,undefined by gcc/g++ into a
temporary directory; the device objects of the regular build are linked
unchanged (GPU code is not sanitized).  Then the oracle pins and the ABI
tests run in a child Python with the sanitizer runtimes preloaded and both
libraries swapped in (AARMS_ORACLE_LIB, AARMS_LIB), and the plain C consumer
runs linked against the sanitized library.  Any report aborts the child."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"
CSRC = os.path.join(ROOT, "activation_add_rmsnorm_amd", "csrc")
OBJS = [os.path.join(ROOT, "_build", s + ".o") for s in ("norm.hip", "norm_resident.hip", "swiglu.hip")]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or shutil.which("g++") is None or _runtime("libasan.so") is None
    or not os.path.isdir(os.path.join(ROCM, "include")),
    reason="needs gcc/g++ with the sanitizer runtimes and the ROCm headers")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    for o in OBJS:
        assert os.path.exists(o), "build the library first (__graft_entry__.build()): %s is missing" % o
    d = tmp_path_factory.mktemp("san")
    oracle_lib = str(d / "liboracle_san.so")
    _run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall", *SAN,
          "-o", oracle_lib, os.path.join(ROOT, "oracle", "aarms_oracle.c"), "-lm"], timeout=300)
    capi_obj = str(d / "capi_san.o")
    _run(["g++", "-O1", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-isystem", os.path.join(ROCM, "include"), *SAN,
          "-c", os.path.join(CSRC, "capi.cpp"), "-o", capi_obj], timeout=300)
    lib = str(d / "libaarms_san.so")
    _run(["g++", "-shared", "-fPIC", *SAN, "-o", lib, capi_obj, *OBJS,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], timeout=300)
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=":".join(p for p in (_runtime("libasan.so"), _runtime("libubsan.so")) if p),
        # the Python interpreter and the HIP runtime are not built with the
        # sanitizers; only reports from the sanitized code are of interest
        ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        AARMS_ORACLE_LIB=oracle_lib,
        AARMS_LIB=lib,
    )
    return dict(dir=d, lib=lib, oracle=oracle_lib, env=env)


def test_oracle_pins_and_abi_under_sanitizers(sanitized):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        "-m", "not gpu"],
                       capture_output=True, text=True, env=sanitized["env"], cwd=ROOT, timeout=1200)
    out = r.stdout[-6000:] + r.stderr[-6000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
    assert " passed" in r.stdout


def test_c_consumer_under_sanitizers(sanitized):
    exe = str(sanitized["dir"] / "c_consumer_san")
    lib_dir = os.path.dirname(sanitized["lib"])
    _run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", *SAN,
          "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
          os.path.join(ROOT, "tests", "c_consumer.c"), "-o", exe,
          sanitized["lib"], "-Wl,-rpath," + lib_dir], timeout=300)
    env = dict(sanitized["env"])
    env.pop("LD_PRELOAD")      # the executable itself links the runtimes
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
