"""CPU oracle of the MoE expert-FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may.  It
shares no code with the HIP library (expert_ffn_layer_gemm_amd) and never
imports it.

Precision: fp32 (NumPy), as the fp32 reference path of the numeric
verification layer in the Qwen3.5-397B-on-Ironwood page (section 6) and the
layer's stated fp32 accumulation.  Every function cites the passage it follows.
Parity status of each function is listed in moe_oracle.py's header.
"""
from .fp8_e4m3 import e4m3_decode, e4m3_encode, e4m3_table, quantize_groups_128  # noqa: F401
from .mx import mx_quantize_rows, mx_dequantize_rows, mx_scale_exponent  # noqa: F401
from .moe_oracle import (  # noqa: F401
    bf16_bits_to_f32, router_logits, topk_softmax, counting_sort, permute_rows,
    expert_ffn, grouped_ffn, combine, forward, forward_tokens, OracleResult, expert_weights_f32,
    quantize_act,
)
