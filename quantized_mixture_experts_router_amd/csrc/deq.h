// In-register decoding of packed weight codes into matrix-core B fragments.
//
// Asymmetric blocks (w = s*q + m; AWQ-style zero point of the "sparse
// activation" page, section 4.4; the per-expert bit widths of the AlphaQ blog,
// section 4.2): a pair of b-bit codes is masked into the mantissas of two
// fp16 numbers with exponent field 25 (value 1024 + q, exact), 1024 is
// subtracted (exact), and one packed fp16 fma applies the group scale and
// minimum (one rounding to fp16).
// e2m1 blocks: placing the three magnitude bits at fp16 bits 9..11 and the
// sign at bit 15 gives exactly v(q) * 2^-14 for all 16 codes (code 1 lands in
// the fp16 subnormal 2^-15 = 0.5 * 2^-14); one exact multiply by 2^14 and one
// multiply by the group scale follow.
#pragma once

#include "common.h"

namespace moeq {

// Global-address-space views: loads through them compile to global_load_*
// (not flat_load_*), which keeps LDS and memory wait counters separate.
#define MOEQ_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ inline const MOEQ_GLOBAL T* gptr(const void* p) {
  return (const MOEQ_GLOBAL T*)(p);
}

__device__ inline f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

template <int EB>
struct PBuf;
template <>
struct PBuf<2> {
  uint32_t w[1];
  __device__ inline void load(const uint8_t* p) { w[0] = *gptr<uint16_t>(p); }
};
template <>
struct PBuf<4> {
  uint32_t w[1];
  __device__ inline void load(const uint8_t* p) { w[0] = *gptr<uint32_t>(p); }
};
template <>
struct PBuf<8> {
  uint32_t w[2];
  __device__ inline void load(const uint8_t* p) {
    u32x2 v = *gptr<u32x2>(p);
    w[0] = v.x;
    w[1] = v.y;
  }
};
template <>
struct PBuf<16> {
  uint32_t w[4];
  __device__ inline void load(const uint8_t* p) {
    u32x4 v = *gptr<u32x4>(p);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
};

// Decode the 8 codes of MFMA step `s` from a lane's 16-byte code block.
template <class F>
__device__ inline f16x8 dequant_step(const u32x4& c, const PBuf<F::EB>& pb, int s) {
  // parameter index inside the entry for lane-local codes [8s, 8s+8)
  const int p = F::kGroup < F::SPAN ? (8 * s) / F::kGroup : 0;
  uint32_t d;
  int base_sh;
  if (F::kBits == 4) {
    d = c[s];
    base_sh = 0;
  } else {
    d = c[s >> 1];
    base_sh = (s & 1) * 8;  // fields 4..7 of the pair sequence start at bit 8
  }
  f16x2 out[4];
  if (F::kFmt == MOE_W_ASYM) {
    const uint32_t sm = pb.w[p];
    const f16x2 s2 = as_f16x2((sm & 0xffffu) * 0x10001u);
    const f16x2 m2 = as_f16x2((sm >> 16) * 0x10001u);
    const f16x2 k1024 = as_f16x2(0x64006400u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t t;
      if (F::kBits == 4)
        t = ((d >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
      else
        t = ((d >> (base_sh + 2 * i)) & 0x00030003u) | 0x64006400u;
      f16x2 q = as_f16x2(t) - k1024;
      out[i] = __builtin_elementwise_fma(q, s2, m2);
    }
  } else {
    const uint32_t sw = (pb.w[p >> 1] >> (16 * (p & 1))) & 0xffffu;
    const f16x2 s2 = as_f16x2(sw * 0x10001u);
    const f16x2 two14 = as_f16x2(0x74007400u);  // 16384.0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t t = d >> (4 * i);
      uint32_t h = ((t & 0x00070007u) << 9) | ((t & 0x00080008u) << 12);
      out[i] = (as_f16x2(h) * two14) * s2;
    }
  }
  f16x8 r;
  r[0] = out[0][0];
  r[1] = out[0][1];
  r[2] = out[1][0];
  r[3] = out[1][1];
  r[4] = out[2][0];
  r[5] = out[2][1];
  r[6] = out[3][0];
  r[7] = out[3][1];
  return r;
}

}  // namespace moeq
