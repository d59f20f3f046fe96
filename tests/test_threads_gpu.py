"""Calls from several host threads at once, each on its own stream.

The library keeps no per-call state outside the call (its only shared
state is a few per-device caches filled with atomic stores), and ctypes
releases the interpreter lock for the duration of a foreign call, so these
calls really overlap in the library.  Every thread's results must equal the
same calls made from one thread.
"""

from __future__ import annotations

import threading

import pytest
import torch

import activation_add_rmsnorm_amd as A

pytestmark = pytest.mark.gpu


def _inputs(seed: int):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = lambda *s: torch.randn(*s, device="cuda", generator=g).to(torch.bfloat16)
    T = 256 + 64 * seed
    return dict(x=bf(T, 4096), r=bf(T, 4096), w=(1 + 0.1 * bf(4096).float()).bfloat16(), gu=bf(T, 2 * 2816),
                scale=torch.tensor([0.03], dtype=torch.float32, device="cuda"))


def _calls(d):
    out, res = A.fused_add_rmsnorm(d["x"], d["r"], d["w"], 1e-6)
    q, s, res2 = A.fused_add_rmsnorm_quant_fp8(d["x"], d["r"], d["w"], 1e-5)
    y = A.swiglu(d["gu"])
    yq = A.swiglu_quant_fp8(d["gu"], d["scale"])
    return [out, res, q, s, res2, y, yq]


def _bits(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_threads_on_separate_streams_match_one_thread():
    n = 4
    data = [_inputs(i) for i in range(n)]
    torch.cuda.synchronize()
    ref = [[_bits(t).clone() for t in _calls(d)] for d in data]
    torch.cuda.synchronize()

    results = [None] * n
    errors = []
    start = threading.Barrier(n)

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                last = None
                for _ in range(20):
                    last = _calls(data[i])
                s.synchronize()
                results[i] = [_bits(t).clone() for t in last]
                s.synchronize()
        except Exception as e:           # reported below, from the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(n):
        for k, (a, b) in enumerate(zip(results[i], ref[i])):
            assert torch.equal(a, b), f"thread {i}, output {k} differs from the single-thread call"
