"""Plain float64 CPU oracle of the MoE-FFN forward and backward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's cpu_baseline leg, never by the HIP library or its binding."""
from . import moe_backward, moe_oracle
from .moe_oracle import (router_logits, softmax, sigmoid_normalized, gate, topk_renorm, renorm,
                         routing, expert_choice_rows,
                         selection_gap, capacity, dispatch, gelu, silu, expert_ffn,
                         combine_rows, aux_stats, routing_stats, forward,
                         e4m3_values, quantize_fp8_rows, dequantize_fp8_rows,
                         expert_choice_select, expert_choice_gap, forward_expert_choice)
