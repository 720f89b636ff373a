"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only *draws* inputs (activations, router weights, packed expert
codes, scales, hash tables, token ids). It contains none of the layer's
arithmetic: no dequantisation, no routing, no matmul. Both the CPU oracle and
the GPU path consume what it produces, so the two sides see bit-identical
inputs while sharing no compute code.
"""
from .configs import (  # noqa: F401
    FormatSpec,
    MoeConfig,
    CONFIGS,
    config,
    variant,
    stack_configs,
)
from .gen import (  # noqa: F401
    QTensor,
    ExpertWeights,
    Layer,
    f32_to_bf16_bits,
    gen_router,
    gen_expert,
    gen_shared,
    gen_routed_stacked,
    gen_layer,
    gen_x,
    gen_token_ids,
    gen_tid2eid,
    gen_bf16_weights,
)
