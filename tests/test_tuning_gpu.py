"""The start-up autotuner on the GPU: every fitting variant is timed, the
report is consistent, a variant it installs is the one the entry points then
run, and results stay equal to the oracle's."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import activation_add_rmsnorm_amd as A
from activation_add_rmsnorm_amd import tuning
from tests import parity as P
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def empty_table():
    tuning.clear()
    yield
    tuning.clear()


def test_sweep_and_tune_report():
    print("[gpu] tuning sweep fused_add_rmsnorm [64,1536]", flush=True)
    times = tuning.sweep("fused_add_rmsnorm", 64, 1536, rounds=2)
    assert set(times) == set(tuning.variants_fitting("fused_add_rmsnorm", 1536))
    assert all(0 < t < 1e4 for t in times.values())
    rep = tuning.tune("swiglu", 16, 8960, rounds=2)
    print("[gpu]", rep, flush=True)
    assert rep["best_us"] <= rep["heuristic_us"]
    assert rep["installed"] in (None, rep["best"])


def test_installed_variant_runs_and_matches_oracle():
    # margin -1: install the fastest whatever the heuristic does
    rep = tuning.tune("fused_add_rmsnorm", 64, 1536, margin=-1.0, rounds=1)
    print("[gpu]", rep, flush=True)
    assert rep["installed"] == rep["best"]
    v = tuning.variant_for("fused_add_rmsnorm", 64, 1536)
    assert A.variant_name(A.OP_NORM, v) == rep["best"]
    x = gen.normal_bf16((64, 1536), 41, 1)
    r = gen.normal_bf16((64, 1536), 41, 2)
    w = gen.normal_bf16((1536,), 41, 3, mean=1.0, std=0.1)
    out, ro = A.fused_add_rmsnorm(P.to_gpu_bf16(x), P.to_gpu_bf16(r), P.to_gpu_bf16(w), 1e-6)
    torch.cuda.synchronize()
    P.check_norm(x, r, w, 1e-6, P.from_gpu_bits(out), P.from_gpu_bits(ro))

    rep = tuning.tune("swiglu_quant_fp8_dynamic", 8, 8960, margin=-1.0, rounds=1)
    print("[gpu]", rep, flush=True)
    gu = gen.normal_bf16((8, 2 * 8960), 42, 4, std=2.0)
    q, s = A.swiglu_quant_fp8_dynamic(P.to_gpu_bf16(gu))
    torch.cuda.synchronize()
    P.check_swiglu_fp8_dynamic(gu, P.from_gpu_bits(q), P.from_gpu_bits(s))
