"""The C ABI from C: tests/c_consumer.c includes include/aarms.h as C11,
links libaarms.so with gcc and runs the argument checks that return before
any HIP call (no GPU needed, no Python between the caller and the library)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import activation_add_rmsnorm_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs gcc and the ROCm headers")
def test_c_program_links_and_sees_documented_statuses(tmp_path):
    lib_dir = os.path.dirname(A.lib_path())
    assert os.path.exists(A.lib_path()), "libaarms.so is not built"
    exe = tmp_path / "c_consumer"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "c_consumer.c"), "-o", str(exe),
           "-L", lib_dir, "-laarms", "-Wl,-rpath," + lib_dir]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout
