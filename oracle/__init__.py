"""fp64 CPU oracle (test infrastructure only; never part of the product path)."""
from .moe_oracle import (  # noqa: F401
    BF16, F32, FP8, combine, decode_activations, expert_capacity, decode_bf16, decode_e4m3fn, decode_matrix,
    expert_down, expert_ffn, ffn, gather_rows, layer, layer_tokens, make_weight_decoder, permute,
    rel_max_err, round_bf16_value, route, router_logits, silu,
)
