"""CPU oracle (test infrastructure only; see bi_oracle's header)."""
from .bi_oracle import *  # noqa: F401,F403
from .bi_oracle import (  # noqa: F401
    bf16_decode, f16_decode, bf16_round, rmsnorm, gemm, int4_codes,
    dequant_int4_g32, gemm_w4, rope, attention_weights, attention,
    decode_attention, residual_add, swiglu, block_forward,
)
