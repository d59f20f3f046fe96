"""The start-up autotuner on the GPU: every fitting variant is timed, the
report is consistent, a variant it installs is the one the entry points then
run, and results stay equal to the oracle's."""

from __future__ import annotations

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


@pytest.mark.parametrize("form", sorted(tuning.FORMS))
def test_every_form_sweeps_every_fitting_variant(form):
    # 2,048 wide: a multiple of every block size (16, 32, 128)
    print("[gpu] tuning sweep", form, "[16,2048]", flush=True)
    times = tuning.sweep(form, 16, 2048, rounds=1)
    assert set(times) == set(tuning.variants_fitting(form, 2048))
    assert all(0 < t < 1e4 for t in times.values())


def test_installed_group_variant_matches_oracle():
    rep = tuning.tune("swiglu_quant_fp8_group", 32, 8960, margin=-1.0, rounds=1)
    print("[gpu]", rep, flush=True)
    assert rep["installed"] == rep["best"]
    gu = gen.normal_bf16((32, 2 * 8960), 43, 4, std=2.0)
    q, s = A.swiglu_quant_fp8_group(P.to_gpu_bf16(gu))
    torch.cuda.synchronize()
    P.check_swiglu_fp8_group(gu, P.from_gpu_bits(q), P.from_gpu_bits(s))

    rep = tuning.tune("fused_add_rmsnorm_quant_fp8_group", 32, 4096, margin=-1.0, rounds=1)
    print("[gpu]", rep, flush=True)
    x = gen.normal_bf16((32, 4096), 44, 1)
    r = gen.normal_bf16((32, 4096), 44, 2)
    w = gen.normal_bf16((4096,), 44, 3, mean=1.0, std=0.1)
    q, s, ro = A.fused_add_rmsnorm_quant_fp8_group(P.to_gpu_bf16(x), P.to_gpu_bf16(r), P.to_gpu_bf16(w), 1e-5)
    torch.cuda.synchronize()
    P.check_norm_fp8_group(x, r, w, 1e-5, P.from_gpu_bits(q), P.from_gpu_bits(s), P.from_gpu_bits(ro))
