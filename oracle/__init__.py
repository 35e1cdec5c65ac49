"""CPU oracle (test infrastructure only; see oracle/oracle.py)."""

from .oracle import (  # noqa: F401
    Oracle,
    apply_rope,
    argmax_first,
    bf16_to_f32,
    f32_to_bf16,
    gqa_attention,
    rmsnorm,
    rope_angles,
    silu,
    softmax,
    swiglu_ffn,
)
