"""The decode-shaped chain -- 28 layers x (fused_add_rmsnorm, fused_add_rmsnorm,
swiglu) on Qwen2.5-1.5B dims -- launched eagerly and captured once per token
count into a HIP graph and replayed.

Checks: every graph replay equals the eager chain bit for bit; the final
residual stream equals the oracle's chain bit for bit; every per-layer output
passes the op's own parity rule.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import activation_add_rmsnorm_amd as A
import oracle
from tests import parity as P
from workloads import configs as W

pytestmark = pytest.mark.gpu


def announce(*what):
    print("[gpu]", *what, flush=True)


class DecodeChain:
    """Static device buffers for one token count, and the 84 launches."""

    def __init__(self, wl: W.DecodeWorkload, T: int, layers: int | None = None):
        self.wl, self.T = wl, T
        self.L = wl.layers if layers is None else layers
        self.host = [W.decode_layer_inputs(wl, T, l) for l in range(self.L)]
        self.res0 = W.decode_residual(wl, T)
        dev = lambda b: P.to_gpu_bf16(b, "cuda")
        self.res = dev(self.res0)
        self.x1 = [dev(h["x1"]) for h in self.host]
        self.x2 = [dev(h["x2"]) for h in self.host]
        self.w1 = [dev(h["w1"]) for h in self.host]
        self.w2 = [dev(h["w2"]) for h in self.host]
        self.gu = [dev(h["gate_up"]) for h in self.host]
        H, N = wl.hidden, wl.inter
        e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
        self.o1 = [e(T, H) for _ in range(self.L)]
        self.o2 = [e(T, H) for _ in range(self.L)]
        self.y = [e(T, N) for _ in range(self.L)]

    def reset(self):
        self.res.copy_(P.to_gpu_bf16(self.res0, "cuda"))

    def step(self):
        eps = self.wl.eps
        for l in range(self.L):
            A.fused_add_rmsnorm(self.x1[l], self.res, self.w1[l], eps, out=self.o1[l], residual_out=self.res)
            A.fused_add_rmsnorm(self.x2[l], self.res, self.w2[l], eps, out=self.o2[l], residual_out=self.res)
            A.swiglu(self.gu[l], out=self.y[l])

    def snapshot(self):
        torch.cuda.synchronize()
        return ([P.from_gpu_bits(t) for t in self.o1], [P.from_gpu_bits(t) for t in self.o2],
                [P.from_gpu_bits(t) for t in self.y], P.from_gpu_bits(self.res))


@pytest.mark.parametrize("T", [1, 8, 32, 128, 256])
def test_decode_chain_graph_vs_eager_vs_oracle(T):
    wl = W.DECODE_GRAPH
    announce("decode chain", "T", T, "layers", wl.layers)
    ch = DecodeChain(wl, T)
    ch.reset()
    ch.step()
    eager = ch.snapshot()

    # oracle: the residual chain and every layer's outputs
    res = ch.res0
    for l in range(ch.L):
        h = ch.host[l]
        P.check_norm(h["x1"], res, h["w1"], wl.eps, eager[0][l], oracle.residual_add(h["x1"], res))
        res = oracle.residual_add(h["x1"], res)
        P.check_norm(h["x2"], res, h["w2"], wl.eps, eager[1][l], oracle.residual_add(h["x2"], res))
        res = oracle.residual_add(h["x2"], res)
        P.check_swiglu(h["gate_up"], eager[2][l])
    assert np.array_equal(eager[3], res), "final residual differs from the oracle chain"

    # capture once, replay several times with eager work and syncs in between
    announce("capture", T)
    ch.reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ch.step()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ch.step()
    for rep in range(3):
        for t in ch.o1 + ch.o2 + ch.y:
            t.fill_(0.0)
        ch.reset()
        torch.cuda.synchronize()
        announce("replay", rep, "T", T)
        g.replay()
        got = ch.snapshot()
        for a, b in zip(eager[0] + eager[1] + eager[2], got[0] + got[1] + got[2]):
            assert np.array_equal(a, b)
        assert np.array_equal(eager[3], got[3])
