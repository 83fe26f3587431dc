"""Seeded synthetic inputs for the W3A16 + low-rank MoE layer.

This module only draws random numbers and lays them out in the shapes of the
workloads; it holds none of the method's arithmetic (no quantization, no
packing, no routing, no matmul).  Both the CPU oracle and the GPU library are
fed from here, so the two always see bit-identical inputs.

Shapes and distributions follow the MiLo setting: Mixtral-8x7B-shaped and
DeepSeekMoE-16B-shaped expert FFNs (the MLSys 2025 talk write-up
"MiLo: Efficient Quantized MoE Inference with Mixture of Low-Rank
Compensators", sections Background and Experimental Setup & Results), with
random weights instead of trained ones.
"""
from .configs import CONFIGS, LinearConfig, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    gen_linear,
    gen_moe_layer,
    gen_logits,
    gen_tokens,
    gen_expert,
    gen_ranks,
    tensor_seed,
)
