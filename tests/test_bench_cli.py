"""bench.py's command line, without a GPU: it measures one GPU only and says
so for any other count, and its byte counts are the algorithmic ones."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes():
    # every input read once, every output written once, the weight once
    T, H, N = 4096, 1536, 8960
    assert bench.norm_bytes(T, H) == T * H * 2 * 4 + H * 2
    assert bench.swiglu_bytes(T, N) == T * N * 2 * 3
    assert bench.norm_bytes(T, H) + bench.swiglu_bytes(T, N) == 270535680


def test_rotation_covers_three_times_the_last_level_cache():
    for b in (25_168_896, 50_334_720, 220_200_960, 234_921_984, 1_174_405_124):
        n = bench.rotation_sets(b)
        assert n >= 2 and n * b >= 3 * bench.MALL_BYTES


def test_configs_filter_parses(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--configs", "llama70b_swiglu"])
    args = bench.parse()
    assert args.configs == "llama70b_swiglu" and args.gpus == 1
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().configs is None


def test_cpu_model_is_named_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
