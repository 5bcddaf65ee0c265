"""Quantized MoE FFN layer for AMD Instinct MI355X (gfx950).

The compute lives in libmoeq.so (hand-written HIP kernels behind the C ABI of
include/moeq.h); this package is its thin Python binding.
"""
from ._lib import (ACT_I8_X, ACT_I8_XH, ACT_NONE, FLAG_BAD_EXPERT_ID, FLAG_NAN_LOGIT, ID_NAN,
                   FLAG_FORMAT_NOT_LAUNCHED, FLAG_BAD_SEGMENT, FLAG_EXPERT_SHAPE, FLAG_FP16_RANGE,
                   MASK_INT8_GEMM, MASK_NO_FUSE, MASK_SHARED_TILE, MASK_OUTLIERS, MASK_SPLIT_GU, MOE_BF16, MOE_F32, MOE_W_ASYM, MOE_W_E2M1, EXPORTED, LIB, LIB_PATH,
                   DeviceQMat, MoeError, PackedExperts, act_quant_i8, combine, expert_histogram, ffn_down,
                   ffn_gather, ffn_gate_up, grouped_ffn, layer_forward, layer_forward_noalloc,
                   noalloc_scratch_bytes, pack_expert, pack_experts,
                   packed_expert_bytes, permute, plan_tiers, read_flags, route, route_i8,
                   route_workspace_size, router_i8_params, router_logit_range,
                   stream_read, stream_read_shaped, version,
                   workspace,
                   workspace_size)

__all__ = [
    "ACT_I8_X", "ACT_I8_XH", "ACT_NONE", "FLAG_BAD_EXPERT_ID", "FLAG_NAN_LOGIT", "ID_NAN",
    "FLAG_FORMAT_NOT_LAUNCHED", "FLAG_BAD_SEGMENT", "FLAG_EXPERT_SHAPE", "FLAG_FP16_RANGE",
    "MASK_INT8_GEMM", "MASK_NO_FUSE", "MASK_SHARED_TILE", "MASK_OUTLIERS", "MASK_SPLIT_GU", "MOE_BF16",
    "MOE_F32", "MOE_W_ASYM", "MOE_W_E2M1", "EXPORTED", "LIB", "LIB_PATH", "DeviceQMat",
    "MoeError", "PackedExperts", "act_quant_i8", "combine", "expert_histogram", "ffn_down",
    "ffn_gather",
    "ffn_gate_up",
    "grouped_ffn", "layer_forward", "layer_forward_noalloc", "noalloc_scratch_bytes", "pack_expert", "pack_experts", "packed_expert_bytes",
    "permute", "plan_tiers", "read_flags", "route", "route_i8", "router_i8_params",
    "router_logit_range", "route_workspace_size", "stream_read", "stream_read_shaped", "version", "workspace", "workspace_size",
]
