"""The Python binding on a GPU: the argument checks name what is wrong, and
the stream handle it passes is the current stream's."""

from __future__ import annotations

import pytest
import torch

import activation_add_rmsnorm_amd as A

pytestmark = pytest.mark.gpu


def test_checks_on_gpu_tensors():
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError, match="dtype"):
        A.fused_add_rmsnorm(x.float(), x, w, 1e-6)
    with pytest.raises(ValueError, match="shape"):
        A.fused_add_rmsnorm(x, x[:, :32].contiguous(), w, 1e-6)
    with pytest.raises(ValueError, match="contiguous"):
        A.fused_add_rmsnorm(x, torch.zeros(64, 4, dtype=torch.bfloat16, device="cuda").t(), w, 1e-6)
    with pytest.raises(ValueError, match="shape"):
        A.fused_add_rmsnorm(x, x, w[:32], 1e-6)
    # a good call still works after the errors
    out, res = A.fused_add_rmsnorm(x, x, w, 1e-6)
    torch.cuda.synchronize()
    assert out.shape == (4, 64) and res.shape == (4, 64)


def test_stream_handle_is_current_stream():
    from activation_add_rmsnorm_amd import _stream
    dev = torch.cuda.current_device()
    assert _stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert _stream(dev) == s.cuda_stream == torch.cuda.current_stream(dev).cuda_stream
    assert _stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    # under capture the handle is the capture stream's
    g = torch.cuda.CUDAGraph()
    x = torch.ones(8, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    res = torch.empty_like(x)
    A.fused_add_rmsnorm(x, x, w, 1e-6, out=out, residual_out=res)
    torch.cuda.synchronize()
    seen = []
    with torch.cuda.graph(g):
        seen.append((_stream(dev), torch.cuda.current_stream(dev).cuda_stream))
        A.fused_add_rmsnorm(x, x, w, 1e-6, out=out, residual_out=res)
    assert seen[0][0] == seen[0][1]
    out.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.all(out == 1.0)


def test_zero_tokens_every_entry_point():
    """Every op on tensors of zero rows (whose data pointers are null): no
    error, no launch, outputs of zero rows; also inside a graph capture, and a
    call with rows still works afterwards."""
    H, N = 1536, 8960
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")
    x, r, gu = bf(0, H), bf(0, H), bf(0, 2 * N)
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    s = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    calls = [
        lambda: A.fused_add_rmsnorm(x, r, w, 1e-6),
        lambda: A.fused_add_rmsnorm_quant_fp8(x, r, w, 1e-6),
        lambda: A.fused_add_rmsnorm_quant_fp8_static(x, r, w, s, 1e-6),
        lambda: A.fused_add_rmsnorm_quant_fp8_group(x, r, w, 1e-6),
        lambda: A.fused_add_rmsnorm_quant_mxfp4(x, r, w, 1e-6),
        lambda: A.fused_add_rmsnorm_quant_nvfp4(x, r, w, s, 1e-6),
        lambda: A.rmsnorm(x, w, 1e-6),
        lambda: A.rmsnorm_quant_fp8(x, w, 1e-6),
        lambda: A.rmsnorm_quant_fp8_static(x, w, s, 1e-6),
        lambda: A.rmsnorm_quant_fp8_group(x, w, 1e-6),
        lambda: A.rmsnorm_quant_mxfp4(x, w, 1e-6),
        lambda: A.rmsnorm_quant_nvfp4(x, w, s, 1e-6),
        lambda: A.swiglu(gu),
        lambda: A.swiglu_quant_fp8(gu, s),
        lambda: A.swiglu_quant_fp8_dynamic(gu),
        lambda: A.swiglu_quant_fp8_group(gu),
        lambda: A.swiglu_quant_mxfp4(gu),
        lambda: A.swiglu_quant_nvfp4(gu, s),
    ]

    def rows(res):
        ts = res if isinstance(res, tuple) else (res,)
        return [t.shape[0] for t in ts]

    for i, c in enumerate(calls):
        assert all(n == 0 for n in rows(c())), i
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        outs = [A.swiglu(gu, out=bf(0, N)), A.fused_add_rmsnorm(x, r, w, 1e-6, out=bf(0, H), residual_out=bf(0, H))]
    torch.cuda.current_stream().wait_stream(st)
    mark = torch.zeros(1, device="cuda")      # one real node, so the graph is not empty
    with torch.cuda.graph(g):
        A.swiglu(gu, out=outs[0])
        A.fused_add_rmsnorm(x, r, w, 1e-6, out=outs[1][0], residual_out=outs[1][1])
        mark.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    assert mark.item() == 1.0
    x1 = torch.ones(2, H, dtype=torch.bfloat16, device="cuda")
    out, res = A.fused_add_rmsnorm(x1, x1, w, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(res, torch.full_like(x1, 2.0)) and torch.equal(out, torch.ones_like(x1))
