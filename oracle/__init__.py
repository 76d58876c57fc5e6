"""CPU oracle (test infrastructure only; see moe_oracle)."""
from .moe_oracle import (  # noqa: F401
    aux_stats, balance_loss, bf16_round, capacity, combine, dequant_rows, dispatch,
    dispatch_next_best, e4m3_decode, expert_choice_capacity, expert_choice_dispatch,
    expert_choice_select, expert_ffn, expert_weights, forward, forward_expert_choice,
    forward_rows, next_best_candidates, renorm_weights, route, router_probs, select_topk,
    silu,
)
