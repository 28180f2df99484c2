"""Seeded synthetic inputs for ProxyAttn prefill attention.

This package only draws random tensors of the shapes and structure the
workloads describe; it contains none of the method's arithmetic (no pooling,
scoring, softmax, budgeting or selection).  Both the CPU oracle and the HIP
path consume its output, so it is the one module they share.
"""
from .configs import CONFIGS, WorkloadConfig, get_config  # noqa: F401
from .generate import (generate, bf16_bits_to_f32, f32_to_bf16_bits, to_bf16_bits,  # noqa: F401
                       input_digest, draw_params)
