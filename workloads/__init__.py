"""Seeded synthetic inputs shaped like the layers of the FP8-RL linear-layer workloads.

This package only draws random tensors (bf16 weights and activations, MoE routing counts). It
contains none of the quantization or GEMM arithmetic, so both the CPU oracle and the HIP path can
take their inputs from it without sharing any of the method's code.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    DENSE_LINEARS_QWEN3_8B,
    LLAMA31_8B_LAYER_LINEARS,
    act_bf16,
    moe_routing_counts,
    moe_expected_padding,
    offsets_from_counts,
    seed_of,
    weight_bf16,
)
