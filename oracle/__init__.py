"""CPU oracle for the MoE layer (test infrastructure only; see mok_oracle)."""
from .mok_oracle import (  # noqa: F401
    Schedule, schedule, dispatch, expert_ffn, combine, silu, sigmoid,
    e4m3_decode, e4m3_encode, mx_scale_exponent, mx_quantize, mx_dequantize, mx_roundtrip,
    bf16_round,
    forward, backward, forward_tokens,
)
