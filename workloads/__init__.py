"""Seeded synthetic workloads shared by the oracle, the tests and the bench.

This package draws random numbers and stores them as bf16 bit patterns.  It
holds none of the arithmetic of the fused operations: the oracle and the GPU
path both consume the bytes it returns and share nothing else.
"""

from .gen import (  # noqa: F401
    bf16_bits_from_f32,
    normal_bf16,
    uniform_f32,
)
from .configs import (  # noqa: F401
    CONFIGS,
    NormWorkload,
    SwigluWorkload,
    DecodeWorkload,
    norm_inputs,
    swiglu_inputs,
    decode_layer_inputs,
    decode_residual,
)
