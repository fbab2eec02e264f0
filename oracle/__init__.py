"""CPU oracle for the sparse MoE layer (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import or call this package. It shares no code with the HIP
library and never imports it.
"""
from .moe import (  # noqa: F401
    backward,
    build,
    capacity_keep,
    combine,
    exp_c,
    expert_capacity,
    expert_choice,
    expert_choice_forward,
    expert_backward,
    expert_fraction,
    expert_forward,
    e4m3_decode,
    e4m3_encode,
    e4m3_round,
    forward,
    forward_mxfp8,
    gate_logits,
    gelu_erf,
    loss_fp64,
    mean_router_probs,
    mx_dequantize,
    mx_quantize,
    mx_roundtrip,
    permutation,
    route,
    router_backward_dlogits,
    router_grads,
    router_losses,
    router_losses_dlogits,
    routing_weights,
    select_topk,
    selection_key,
    sigmoid_c,
    sigmoid_c_sweep,
    silu,
)
