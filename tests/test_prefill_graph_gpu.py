"""Prefill-shaped launches captured into one HIP graph and replayed.

The kernels that order their memory traffic by time -- the bf16 norm of one
wave per row that holds its stores on the real-time clock ([4096, 1536]),
and the resident-row norms that keep a 16,384-wide row in one wave's
registers ([2048, 16384] per-token and per-tensor E4M3 and bf16; [1024,
16384] per-token E4M3 with y kept in place) -- plus the SwiGLU of the same
layer, captured once through torch.cuda.CUDAGraph (a hipGraph).  Between
replays the outputs are overwritten eagerly and the device synchronized;
every replay must then reproduce the eager launches' outputs bit for bit.
Parity of the same launches against the oracle is covered by the parity
tests; this checks that capture and replay change nothing.
"""

from __future__ import annotations

import pytest
import torch

import activation_add_rmsnorm_amd as A

pytestmark = pytest.mark.gpu


def announce(*what):
    print("[gpu]", *what, flush=True)


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32) if t.element_size() == 4 else t


def test_prefill_launches_graph_replay_equals_eager():
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    bf = lambda *s, std=1.0: (torch.randn(*s, device=dev, generator=g) * std).to(torch.bfloat16)
    outs = {}
    ins = {}

    # inputs; every output has its own buffer, so each replay starts from the same state
    ins["n_x"], ins["n_r"], ins["n_w"] = bf(4096, 1536), bf(4096, 1536), (1 + bf(1536, std=0.1).float()).bfloat16()
    ins["s_gu"] = bf(4096, 2 * 8960)
    ins["q_x"], ins["q_r"] = bf(2048, 16384), bf(2048, 16384)
    ins["q_w"] = (1 + bf(16384, std=0.1).float()).bfloat16()
    ins["q1_x"], ins["q1_r"] = bf(1024, 16384), bf(1024, 16384)
    ins["scale"] = torch.tensor([0.02], dtype=torch.float32, device=dev)
    e = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device=dev)
    outs["n_out"], outs["n_res"] = e(4096, 1536), e(4096, 1536)
    outs["s_y"] = e(4096, 8960)
    outs["q_q"], outs["q_s"], outs["q_res"] = e(2048, 16384, dt=torch.uint8), e(2048, dt=torch.float32), e(2048, 16384)
    outs["st_q"], outs["st_res"] = e(2048, 16384, dt=torch.uint8), e(2048, 16384)
    outs["b_out"], outs["b_res"] = e(2048, 16384), e(2048, 16384)
    outs["q1_q"], outs["q1_s"], outs["q1_res"] = e(1024, 16384, dt=torch.uint8), e(1024, dt=torch.float32), e(1024, 16384)

    def launches():
        A.fused_add_rmsnorm(ins["n_x"], ins["n_r"], ins["n_w"], 1e-6, out=outs["n_out"], residual_out=outs["n_res"])
        A.swiglu(ins["s_gu"], out=outs["s_y"])
        A.fused_add_rmsnorm_quant_fp8(ins["q_x"], ins["q_r"], ins["q_w"], 1e-5, out=outs["q_q"],
                                      scale_out=outs["q_s"], residual_out=outs["q_res"])
        A.fused_add_rmsnorm_quant_fp8_static(ins["q_x"], ins["q_r"], ins["q_w"], ins["scale"], 1e-5,
                                             out=outs["st_q"], residual_out=outs["st_res"])
        A.fused_add_rmsnorm(ins["q_x"], ins["q_r"], ins["q_w"], 1e-5, out=outs["b_out"], residual_out=outs["b_res"])
        A.fused_add_rmsnorm_quant_fp8(ins["q1_x"], ins["q1_r"], ins["q_w"], 1e-5, out=outs["q1_q"],
                                      scale_out=outs["q1_s"], residual_out=outs["q1_res"])

    def poison():
        for t in outs.values():
            t.view(torch.uint8).fill_(0xA5)

    announce("prefill graph: eager launches")
    poison()
    launches()
    torch.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in outs.items()}

    announce("prefill graph: capture")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launches()               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        launches()
    torch.cuda.synchronize()

    for rep in range(3):
        announce("prefill graph: replay", rep)
        poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bits(v), ref[k]), f"replay {rep}: {k} differs from the eager launch"
