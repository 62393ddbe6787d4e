"""Seeded synthetic inputs for the grouped expert MLP.

This package only draws random numbers and shapes them into the arrays that
both the GPU path and the CPU oracle consume (routing choices, activations,
weights, upstream gradients).  It holds none of the layer's arithmetic: no
permutation, no quantization, no GEMM, no activation function.
"""
from .configs import CONFIGS, MoEConfig, get_config
from .generate import MoEInputs, make_inputs, make_logits, route_topk

__all__ = ["CONFIGS", "MoEConfig", "get_config", "MoEInputs", "make_inputs", "make_logits", "route_topk"]
