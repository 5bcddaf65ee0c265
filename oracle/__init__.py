"""CPU oracle of the quantized MoE FFN layer forward pass.

TEST INFRASTRUCTURE ONLY. This package is imported by the tests, by the smoke
check and by the benchmark's CPU-baseline leg; the library and its Python
binding never import, call or link it, and it shares no code with them.

It is plain, slow and meant to be checked by eye against the method's
statement: fp64 router logits, an exact stable top-k, a softmax over the
selected logits, a stable counting-sort permutation, blocks decoded to fp32,
fp64 matmuls and an fp64 weighted combine; also the routing histogram and
the precision-tier plan of expert-aware quantisation, and the int8 router
logits with their calibration.
"""
from .moe import (decode_qmat, router_logits, topk_softmax, canonical_permute,
                  act_quant_i8, dq8, swiglu, expert_ffn, combine, moe_layer,
                  x_to_f64, expert_histogram, plan_tiers, router_logit_range,
                  router_i8_params, quantize_logits_i8, topk_softmax_i8, NEAR_TIE, E2M1_TABLE)

__all__ = ["decode_qmat", "router_logits", "topk_softmax", "canonical_permute",
           "act_quant_i8", "dq8", "swiglu", "expert_ffn", "combine", "moe_layer",
           "x_to_f64", "expert_histogram", "plan_tiers", "router_logit_range",
           "router_i8_params", "quantize_logits_i8", "topk_softmax_i8", "NEAR_TIE", "E2M1_TABLE"]
