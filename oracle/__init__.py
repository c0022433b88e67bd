"""Oracle for the MoE FFN layer (test infrastructure only; never imported by
the product path)."""
from .moe_oracle import (bf16_to_f32, bf16_to_f64, router_logits, softmax32, topk, route,
                         dispatch, gather, swiglu, grouped_ffn, shared_experts, combine,
                         moe_layer, token_outputs, expert_node)
