"""CPU oracle of the OLMoE MoE feed-forward layer (float64, NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the GPU library or its binding.
"""
from .moe_ref import (  # noqa: F401
    ALPHA, BETA, RMS_EPS, to_f64, round_to_bf16, bf16_bits, router_logits, softmax_all,
    top_k, mask_logits, renormalize_top_k, dispatch, silu, swiglu_expert, losses, moe_layer_ref, moe_layer_dense_ref,
    rmsnorm_bf16, moe_stack_ref, silu_grad, moe_layer_backward_ref, expert_capacity,
    expert_choice_select, expert_choice_layer_ref, expert_choice_backward_ref,
)
