"""CPU oracle for the batch-1 decode step (test infrastructure only; see decode.py)."""
from .decode import (  # noqa: F401
    apply_rope,
    attend_one_head,
    bf16_to_float,
    decode_step,
    float_to_bf16,
    gemv,
    greedy_decode,
    widen_weights,
    rms_norm,
    rope_cos_sin,
    silu,
)
