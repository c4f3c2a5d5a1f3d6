"""Plain fp64 CPU oracle of the Mixtral-style sparse MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the graft entry
point and the CPU-baseline leg of the benchmark may import this package.  The
product path (the HIP library and its Python binding) never calls it and shares
no code with it.
"""
from .moe_oracle import (  # noqa: F401
    Q4_GROUP,
    bf16_round,
    brute_force_topk,
    capacity_dispatch,
    dequantize_q4,
    dispatch,
    expert_capacity,
    expert_choice_capacity,
    expert_choice_dispatch,
    expert_choice_select,
    expert_swiglu,
    forward,
    forward_capacity,
    forward_expert_choice,
    forward_kept,
    forward_mask_form,
    forward_with_selection,
    full_softmax,
    gate_weights,
    mixtral_param_counts,
    quantize_q4,
    route,
    router_logits,
    router_stats,
    sigmoid,
    silu,
    topk_select,
    unpack_q4,
)
