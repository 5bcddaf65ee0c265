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
// 8 int8 codes (integral fp32 values in [-127, 127]) in the byte order of
// the int8 GEMM's operands: byte p holds code perm8(p), perm8 = 0,4,1,5,2,6,3,7,
// the order in which a 4-bit weight word's nibbles unpack to bytes. Returns
// their sum.
__device__ inline float store8_i8p(int8_t* dst, const float* q) {
  const int b[8] = {(int)q[0], (int)q[4], (int)q[1], (int)q[5],
                    (int)q[2], (int)q[6], (int)q[3], (int)q[7]};
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    lo |= (uint32_t)(b[p] & 0xff) << (8 * p);
    hi |= (uint32_t)(b[p + 4] & 0xff) << (8 * p);
  }
  *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
  return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

// Sum of one 64-column block over the 8 lanes holding it (lanes 8j..8j+7 of
// a wavefront, 8 columns each); stored by the first of them into the int8
// GEMM's tile-major sums: sums[(c / 128) R + r][(c / 64) % 2].
__device__ inline void store_sum64(float* sums, int R, int r, int c, float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  if ((threadIdx.x & 7) == 0) sums[((size_t)(c >> 7) * R + r) * 2 + ((c >> 6) & 1)] = v;
}

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
