"""CPU oracle of the MoE layer (float64, numpy).

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (  # noqa: F401
    E2M1_MAGNITUDE, NEAR_TIE, bf16_to_f64, build_permutation, combine, expert_ffn, forward,
    gate_weights, gpt_oss_param_counts, mxfp4_bits_per_param, mxfp4_decode, round_to_bf16,
    router_logits, select_experts, silu, swiglu, rms_norm, block_forward, f64_to_bf16_bits,
    mxfp4_quantize_rows,
)
