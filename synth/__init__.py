"""Seeded synthetic inputs for the quantized MoE FFN layer.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle. It draws inputs and writes weight blobs in the canonical block format;
it holds none of the layer's forward arithmetic (no decoding, no router, no
top-k, no matmul).

Sources for the shapes and distributions (the workloads of the pages, drawn
synthetically because no trained weights or datasets are available):
  * Mixtral-8x7B expert shapes (hidden 4096, 8 experts, top-2, intermediate
    14336): "AlphaQ" blog, sections 1 and 3.
  * 256 routed experts, top-6, 4-bit floating-point (NVFP4-style) weights:
    Baidu Cloud article on a quantized MoE LLM, "expert routing" section.
  * 64 hot experts at 4-bit / 192 cold experts at 2-bit, and the routing skew
    "top 32 of 256 experts take about half of the routes": expert-aware
    quantisation digest, profiling and results sections.
  * per-token dynamic int8 expert inputs: MoE mixed-precision field notes,
    section 2.1.

Weights of the large workloads are drawn directly as codes plus per-group
parameters whose value ranges match a 4-/2-bit asymmetric (or e2m1)
quantisation of N(0, 0.02) weights; quantising tens of billions of Gaussian
draws in NumPy would dominate every run. The tiny workload goes through the
real quantiser.
"""
from .formats import (FMT_ASYM, FMT_E2M1, QMat, quantize_asym, quantize_e2m1,
                      random_qmat, row_bytes, f32_to_bf16_bits, bf16_bits_to_f32,
                      E2M1_VALUES)
from .configs import (LayerConfig, CONFIGS, get_config, gen_router, gen_x,
                      gen_expert, expert_format, matrix_formats, scaled_config)

__all__ = [
    "FMT_ASYM", "FMT_E2M1", "QMat", "quantize_asym", "quantize_e2m1",
    "random_qmat", "row_bytes", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "E2M1_VALUES", "LayerConfig", "CONFIGS", "get_config", "gen_router",
    "gen_x", "gen_expert", "expert_format", "matrix_formats", "scaled_config",
]
