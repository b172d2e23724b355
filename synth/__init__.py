"""Seeded synthetic inputs for the gpt-oss MoE feed-forward layer.

This package is shared by the CPU oracle tests and the GPU path. It holds
input preparation only: random draws, bf16 rounding of the activations and
the MXFP4 *encoder* that turns fp32 weights into the packed bytes both sides
read. It performs none of the layer's arithmetic (no routing, no decode, no
expert evaluation) and imports neither the oracle nor the HIP library.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    RMS_NORM_EPS,
    SWIGLU_LIMIT,
    LayerInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    mxfp4_encode,
)
