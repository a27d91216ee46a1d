"""Seeded synthetic inputs for block-sparse attention with pooled block routing.

This package only draws random tensors of the shapes and structure of the
workloads the method is aimed at (DiT image/video attention, long-context LLM
prefill).  It contains none of the method's arithmetic, so the CPU oracle's
tests and the GPU path's tests/bench can both take their inputs from here.
"""

from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits,
    bf16_round,
    get_config,
    make_group,
    make_inputs,
    output_gradient,
    random_qkv,
)
