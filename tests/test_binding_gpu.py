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
