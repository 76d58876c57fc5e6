"""CPU oracle (test infrastructure only; see moe_oracle)."""
from .moe_oracle import (  # noqa: F401
    aux_stats, balance_loss, bf16_round, capacity, combine, dequant_rows, dispatch,
    e4m3_decode, expert_ffn, expert_weights, forward, forward_rows, renorm_weights, route,
    router_probs, select_topk, silu,
)
