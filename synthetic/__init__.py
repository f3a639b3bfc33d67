"""Seeded synthetic inputs for the decoder forward pass.

This package is the only code shared by the CPU oracle (``oracle/``) and the
GPU path's tests and benchmark. It draws model weights, prompts and context
lengths from fixed seeds and holds none of the forward pass's arithmetic:
no normalisation, rotation, attention, dequantisation or matrix product.

Model shapes follow the Qwen3-0.6B layout described on the pages
("A real model in our own decoder", section "Same design, bigger numbers,
five switches") and a two-layer tiny decoder with the same switches.
"""

from .configs import MODELS, WORKLOADS, ModelShape, param_count
from .generate import (
    Weights,
    make_weights,
    make_prompts,
    make_context_lengths,
    fp32_to_bf16_bits,
    quantize_uint4_g32,
    quantize_int4_sym_g32,
)

__all__ = [
    "MODELS",
    "WORKLOADS",
    "ModelShape",
    "param_count",
    "Weights",
    "make_weights",
    "make_prompts",
    "make_context_lengths",
    "fp32_to_bf16_bits",
    "quantize_uint4_g32",
    "quantize_int4_sym_g32",
]
