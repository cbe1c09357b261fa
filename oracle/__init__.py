"""FP64 CPU oracle of the top-k MoE SwiGLU layer -- test infrastructure only.

Imported only by the tests, the package smoke check and the benchmark's
CPU-baseline leg; the HIP library never imports, links or calls it.
Every function is pinned by the CPU test suite (no function here is
"parity unpinned")."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (INT4_GROUP, assign_rows, bf16_to_f64, capacity_rows,  # noqa: F401
                         experts_touched_expected, f32_to_f64, fp8_dequant, fp8_e4m3_to_f64,
                         gate_weights, int4_dequant, limit_groups,
                         int4_unpack, moe_layer, router_logits, select_topk, sigmoid_scores,
                         silu, softmax_scores, swaps_per_token, swiglu_ffn, round_to_bf16,
                         round_to_e4m3, quantize_rows_e4m3, dequant_rows_e4m3, swiglu_ffn_a8)
