"""The workloads the fused ops are measured and checked on.

The shapes stand in for the layers the pages run: Qwen2.5-1.5B-Instruct
(hidden 1,536, MLP intermediate 8,960, 28 layers, two RMSNorms and one gated
MLP per layer; "TensorRT-LLM: Compiling Inference Engines Ahead of Time",
section "Fusing operations, measured") and the Llama 3.1 FP8 setting of the
vLLM torch.compile post (section 4, experiments).  No weights or datasets
are used: every tensor is a seeded draw from ``gen``.
"""

from __future__ import annotations

from dataclasses import dataclass

from .gen import normal_bf16

# Sub-stream ids: one per tensor role, so that each tensor's bytes are fixed
# by (seed, role) alone.
ID_X = 1
ID_RESIDUAL = 2
ID_WEIGHT = 3
ID_GATE_UP = 4


def _decode_id(layer: int, role: int) -> int:
    # roles: 0 = x of the first norm, 1 = x of the second norm,
    #        2 = weight of the first norm, 3 = weight of the second, 4 = gate_up
    return 1000 + 10 * layer + role


@dataclass(frozen=True)
class NormWorkload:
    """fused_add_rmsnorm (optionally with per-token FP8) on bf16 [tokens, hidden]."""
    name: str
    tokens: int
    hidden: int
    eps: float
    seed: int = 0
    outlier_frac: float = 0.0
    outlier_mult: float = 50.0
    quant_fp8: bool = False


@dataclass(frozen=True)
class SwigluWorkload:
    """swiglu (optionally with static FP8) on bf16 gate_up [tokens, 2*inter]."""
    name: str
    tokens: int
    inter: int
    gate_up_std: float = 1.0
    seed: int = 0
    quant_fp8: bool = False
    scale: float | None = None


@dataclass(frozen=True)
class DecodeWorkload:
    """A decode step's memory-bound chain: layers x (2 norms + 1 swiglu)."""
    name: str
    tokens: tuple = (1, 8, 32, 128, 256)
    layers: int = 28
    hidden: int = 1536
    inter: int = 8960
    eps: float = 1e-6
    seed: int = 0


NORM_DECODE16 = NormWorkload("qwen1.5b_norm_16x1536", tokens=16, hidden=1536, eps=1e-6)
NORM_PREFILL4096 = NormWorkload("qwen1.5b_norm_4096x1536", tokens=4096, hidden=1536, eps=1e-6)
SWIGLU_PREFILL4096 = SwigluWorkload("qwen1.5b_swiglu_4096x17920", tokens=4096, inter=8960)
DECODE_GRAPH = DecodeWorkload("qwen1.5b_decode_28layers")
SWIGLU_FP8_LLAMA70B = SwigluWorkload("llama70b_swiglu_fp8_8192x57344", tokens=8192, inter=28672,
                                     gate_up_std=2.0, quant_fp8=True, scale=0.05)
NORM_FP8_LLAMA405B = NormWorkload("llama405b_norm_fp8_2048x16384", tokens=2048, hidden=16384,
                                  eps=1e-5, outlier_frac=0.001, outlier_mult=50.0, quant_fp8=True)

# One GPU's share of the two Llama layers when the path is sharded over 8
# GPUs: the norm under sequence parallelism runs on T/8 rows, the SwiGLU under
# tensor parallelism on a [gate_shard | up_shard] of N/8 columns each.
NORM_FP8_LLAMA405B_SP8 = NormWorkload("llama405b_norm_fp8_sp8_256x16384", tokens=256, hidden=16384,
                                      eps=1e-5, outlier_frac=0.001, outlier_mult=50.0, quant_fp8=True)
SWIGLU_FP8_LLAMA70B_TP8 = SwigluWorkload("llama70b_swiglu_fp8_tp8_8192x7168", tokens=8192, inter=3584,
                                         gate_up_std=2.0, quant_fp8=True, scale=0.05)
SHARDS = (NORM_FP8_LLAMA405B_SP8, SWIGLU_FP8_LLAMA70B_TP8)

# name -> the ops of that workload, in the order they run
CONFIGS = {
    "norm_decode16": (NORM_DECODE16,),
    "qwen_prefill4096": (NORM_PREFILL4096, SWIGLU_PREFILL4096),
    "qwen_decode_graph": (DECODE_GRAPH,),
    "llama70b_swiglu_fp8": (SWIGLU_FP8_LLAMA70B,),
    "llama405b_norm_fp8": (NORM_FP8_LLAMA405B,),
}


def norm_inputs(wl: NormWorkload, tokens: int | None = None, hidden: int | None = None) -> dict:
    """x, residual [tokens, hidden] and weight [hidden] as bf16 bit patterns.

    ``tokens``/``hidden`` override the workload's shape (same recipe), for
    scaled-down parity cases.
    """
    t = wl.tokens if tokens is None else int(tokens)
    h = wl.hidden if hidden is None else int(hidden)
    x = normal_bf16((t, h), wl.seed, ID_X, outlier_frac=wl.outlier_frac, outlier_mult=wl.outlier_mult)
    r = normal_bf16((t, h), wl.seed, ID_RESIDUAL, outlier_frac=wl.outlier_frac,
                    outlier_mult=wl.outlier_mult)
    w = normal_bf16((h,), wl.seed, ID_WEIGHT, mean=1.0, std=0.1)
    return {"x": x, "residual": r, "weight": w}


def swiglu_inputs(wl: SwigluWorkload, tokens: int | None = None, inter: int | None = None) -> dict:
    """gate_up [tokens, 2*inter] (gate columns first, then up) as bf16 bits."""
    t = wl.tokens if tokens is None else int(tokens)
    n = wl.inter if inter is None else int(inter)
    gu = normal_bf16((t, 2 * n), wl.seed, ID_GATE_UP, std=wl.gate_up_std)
    return {"gate_up": gu}


def decode_layer_inputs(wl: DecodeWorkload, tokens: int, layer: int) -> dict:
    """Per-layer tensors of the decode chain: distinct x / weight / gate_up per
    layer (stand-ins for the omitted GEMM outputs), all ~N(0,1), weights
    1+N(0,0.1)."""
    h, n = wl.hidden, wl.inter
    return {
        "x1": normal_bf16((tokens, h), wl.seed, _decode_id(layer, 0)),
        "x2": normal_bf16((tokens, h), wl.seed, _decode_id(layer, 1)),
        "w1": normal_bf16((h,), wl.seed, _decode_id(layer, 2), mean=1.0, std=0.1),
        "w2": normal_bf16((h,), wl.seed, _decode_id(layer, 3), mean=1.0, std=0.1),
        "gate_up": normal_bf16((tokens, 2 * n), wl.seed, _decode_id(layer, 4)),
    }


def decode_residual(wl: DecodeWorkload, tokens: int):
    """The residual stream the decode chain starts from, ~N(0,1)."""
    return normal_bf16((tokens, wl.hidden), wl.seed, ID_RESIDUAL)
