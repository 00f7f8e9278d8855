"""CPU oracle (fp64) of the int4-g64 MoE layer and of grouped-query decode attention.
Test infrastructure only: imported by tests, the smoke check and the benchmark's CPU
baseline, never by the library."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (bf16_to_f64, unpack_codes, dequantize, router_logits, select_topk,
                         expert_histogram, group_offsets, stable_permutation, silu, swiglu,
                         grouped_gemm_q4, expert_ffn, combine, moe_layer, moe_out_for_tokens)
from .attention_oracle import gqa_decode_attention  # noqa: F401
