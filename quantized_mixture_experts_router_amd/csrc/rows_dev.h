// Row helpers shared by the expert-input gather kernels: element loads of
// bf16/fp32 rows and the per-token int8 quantiser (mixed-precision notes,
// sections 2.1-2.2: expert inputs quantised per token at run time with an
// absmax scale).
#pragma once

#include "common.h"

namespace moeq {
namespace rows {

__device__ inline float load_val(const void* x, int dt, size_t idx) {
  if (dt == MOE_BF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[idx] << 16);
  return ((const float*)x)[idx];
}

// q = clamp(rint(v / s), -127, 127) with IEEE fp32 division; s = absmax / 127.
__device__ inline float quant_i8(float v, float s) {
  if (s == 0.f) return 0.f;
  float q = __builtin_rintf(__fdiv_rn(v, s));
  return fminf(fmaxf(q, -127.f), 127.f);
}

// 8 consecutive elements of a bf16 or fp32 row as fp32 (16-/32-byte loads)
__device__ inline void load8(const void* x, int dt, size_t idx, float* v) {
  if (dt == MOE_BF16) {
    const u32x4 u = *reinterpret_cast<const u32x4*>((const uint16_t*)x + idx);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(u[q] << 16);
      v[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>((const float*)x + idx);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  }
}

// stores 8 values as fp16; true when one of them is beyond the fp16 range
// (|v| > 65504: stored as +-inf)
__device__ inline bool store8_f16(f16* dst, const float* v) {
  f16x8 h;
  bool over = false;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    h[q] = (f16)v[q];
    over |= fabsf(v[q]) > 65504.0f;
  }
  *reinterpret_cast<f16x8*>(dst) = h;
  return over;
}

}  // namespace rows
}  // namespace moeq
