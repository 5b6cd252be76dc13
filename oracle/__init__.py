"""Float64 CPU oracle for fused scaled dot-product attention (test infrastructure only)."""
from .sdpa_oracle import (  # noqa: F401
    MASK_KINDS,
    attention_weights,
    brute_force_sdpa,
    gather_strided,
    mask_bias,
    merge_states,
    partial_state,
    rope,
    rope_tables,
    sdpa,
    sdpa_strided,
)
