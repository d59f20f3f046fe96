"""The Python binding's argument checks that need no GPU: every op rejects a
non-tensor and a tensor that is not on a GPU before anything reaches the
library (there is no CPU path)."""

from __future__ import annotations

import pytest
import torch

import activation_add_rmsnorm_amd as A


def _cpu(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def test_norm_rejects_cpu_tensors():
    x, r, w = _cpu(4, 64), _cpu(4, 64), _cpu(64)
    with pytest.raises(ValueError, match="GPU"):
        A.fused_add_rmsnorm(x, r, w, 1e-6)
    with pytest.raises(ValueError, match="GPU"):
        A.rmsnorm(x, w, 1e-6)
    with pytest.raises(ValueError, match="GPU"):
        A.fused_add_rmsnorm_quant_fp8(x, r, w, 1e-6)


def test_swiglu_rejects_cpu_tensors():
    with pytest.raises(ValueError, match="GPU"):
        A.swiglu(_cpu(4, 128))
    with pytest.raises(ValueError, match="GPU"):
        A.swiglu_quant_fp8(_cpu(4, 128), torch.tensor([0.05]))


def test_rejects_non_tensors():
    from activation_add_rmsnorm_amd import _require
    with pytest.raises(TypeError, match="torch.Tensor"):
        _require([[0.0] * 64] * 4, "x", (torch.bfloat16,), (4, 64))
    with pytest.raises(TypeError, match="torch.Tensor"):
        _require(None, "weight", (torch.bfloat16,), (64,))
