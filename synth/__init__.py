"""Seeded synthetic inputs for the routed-expert MoE step.

This package only draws random numbers and shapes them into the inputs of the
step (fp32 expert weights, fp32 router matrices, bf16 tokens, router biases, and
the parameters and inputs of the DeltaNet and attention decode steps).
It holds none of the method's arithmetic: no quantisation, routing, expert
math or pool policy. Both the HIP path (through its tests and benchmark) and
the CPU oracle take their inputs from here, and from nowhere else.
"""
from .workload import (  # noqa: F401
    CONFIGS,
    Config,
    get_config,
    expert_weights,
    shared_expert_weights,
    router_weight,
    router_bias,
    shared_gate,
    tokens,
    SynthWeights,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    GDN_CONFIGS,
    GdnConfig,
    get_gdn_config,
    gdn_params,
    gdn_inputs,
    ATTN_CONFIGS,
    AttnConfig,
    get_attn_config,
    attn_params,
    attn_cache,
    attn_inputs,
)
