// In-register decoding of packed weight codes into matrix-core B fragments.
//
// Asymmetric blocks (w = s*q + m; AWQ-style zero point of the "sparse
// activation" page, section 4.4; the per-expert bit widths of the AlphaQ blog,
// sections 2.2 and 4.2; 1-bit for the coldest experts, the sub-2-bit tier of
// the expert-aware quantisation digest's conclusion): a pair of b-bit codes is
// OR-ed into the mantissas of two fp16 numbers (exact), the fp16 offset is
// subtracted (exact), and one packed fp16 fma applies the group scale and
// minimum (one rounding to fp16). 3-bit codes come as a 2-bit plane and a
// 1-bit plane: each gives an exact fp16 pair, and q = q2 + 4 q1 is formed
// exactly before the same fma.
// e2m1 blocks (the 4-bit floating-point weights of the quantized-MoE
// article): the gfx950 fp4 converter yields the exact fp16 value of each code,
// then one fp16 multiply by the group scale (one rounding).
#pragma once

#include "common.h"

namespace moeq {

__device__ inline f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Buffer-resource loads: base and size in scalar registers, a 32-bit
// per-lane offset and a scalar per-tile offset, so a load costs no vector
// address arithmetic. AUX holds the cache-policy bits: 0 (cached) or kNT,
// the non-temporal hint for data read once per call (the decode GEMVs'
// weight streams), which sustains a higher HBM read rate.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kNT = 2;

// a pointer every lane holds, moved to scalar registers
template <class T>
__device__ inline T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}
// descriptor of `bytes` bytes at p (raw buffer: no stride, no format);
// loads past the end return zero
// A buffer offset past every range this library builds (ranges stay below
// 2 GiB): loads at it return zeros without a memory access.
constexpr uint32_t kPastRange = 0x80000000u;
__device__ inline rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
template <class T, int AUX = 0>
__device__ inline T bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 16) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
  } else if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
  } else {
    static_assert(sizeof(T) == 2, "load size");
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX));
  }
}

// One lane's codes of a tile: one load, or two for the 3-bit planes (v: the
// lane's offset in the first plane, vh: in the high-bit plane).
template <class F, int AUX = 0>
__device__ inline typename F::CodeT load_codes(rsrc_t r, uint32_t v, uint32_t vh, uint32_t soff) {
  if constexpr (F::kBits == 3) {
    Codes3 c;
    c.lo = bload<u32x4, AUX>(r, v, soff);
    c.hi = bload<u32x2, AUX>(r, vh, soff);
    return c;
  } else {
    return bload<typename F::CodeT, AUX>(r, v, soff);
  }
}
// loads a load_codes call issues
template <class F>
constexpr int code_loads() { return F::kBits == 3 ? 2 : 1; }

// Block parameters of one lane's codes (EB bytes: fp16 scale, or scale and
// minimum, for one or two groups), zero-extended into 32-bit words.
template <int EB>
struct PBuf {
  static_assert(EB == 2 || EB == 4 || EB == 8 || EB == 16, "parameter bytes");
  uint32_t w[EB <= 4 ? 1 : EB / 4];
  template <int AUX = 0>
  __device__ inline void load(rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (EB == 2) {
      w[0] = bload<uint16_t, AUX>(r, voff, soff);
    } else if constexpr (EB == 4) {
      w[0] = bload<uint32_t, AUX>(r, voff, soff);
    } else if constexpr (EB == 8) {
      const u32x2 v = bload<u32x2, AUX>(r, voff, soff);
      w[0] = v.x;
      w[1] = v.y;
    } else {
      const u32x4 v = bload<u32x4, AUX>(r, voff, soff);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    }
  }
};

// Constants of the decoders, held in VGPRs for the whole kernel: gfx9 VOP3
// encodings take no literal operand, so v_and_or_b32 needs its mask and its
// exponent pattern in registers. `opaque` stops the compiler from folding
// them back into literals.
__device__ inline uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Asymmetric b-bit codes: within a 32-bit word the pair (code 2i, code 2i+1)
// sits in the two 16-bit halves at the same bit offset o = b*i (mod 8 after a
// shift by 8 for the upper pairs). OR-ing the masked field into the mantissa
// of an fp16 number whose last mantissa bit weighs 2^-o, i.e. 2^(10-o), gives
// exactly 2^(10-o) + q; subtracting 2^(10-o) leaves q.
struct DeqConsts {
  uint32_t mask[4];    // field masks for offsets 0, b, 2b, 3b (b = bits), both halves
  uint32_t magic[4];   // fp16 pairs 2^(10 - offset)
  uint32_t mask_h[4];  // 3-bit: the high-bit plane's fields at offsets 0..3
  uint32_t magic_h[4]; // 3-bit: fp16 pairs 2^(12 - offset), so a set bit adds 4
};

template <class F>
__device__ inline DeqConsts make_deq_consts() {
  DeqConsts k;
  // 3-bit codes decode their low two bits as a 2-bit plane
  constexpr int B = F::kBits == 3 ? 2 : F::kBits;
  const uint32_t fm = (1u << B) - 1u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int off = B * j;
    const bool used = F::kFmt == MOE_W_ASYM && (B <= 2 || j < 2);
    const uint32_t mk = ((fm << off) | (fm << (16 + off)));
    const uint32_t e = 25u - off;  // fp16 exponent field of 2^(10 - off)
    const uint32_t mg = (e << 10) | (e << 26);
    k.mask[j] = used ? opaque(mk) : 0u;
    k.magic[j] = used ? opaque(mg) : 0u;
    // high bit of a 3-bit code at offset j of its plane: 2^(12 - j) + 4 q1
    const uint32_t eh = 27u - j;
    k.mask_h[j] = F::kBits == 3 ? opaque((1u << j) | (1u << (16 + j))) : 0u;
    k.magic_h[j] = F::kBits == 3 ? opaque((eh << 10) | (eh << 26)) : 0u;
  }
  return k;
}

// -(2^(12 - j) + 2^(10 - 2j)) in both halves (exact in fp16: at most six
// significant bits): subtracting it from the high-bit pair and adding the
// low-two-bit pair leaves q = q2 + 4 q1 exactly
__device__ inline f16x2 magic3_sub(int j) {
  const f16 c = (f16)(-(float)((1 << (12 - j)) + (1 << (10 - 2 * j))));
  return f16x2{c, c};
}

__device__ inline f16x2 magic_sub(int off) {
  // -(2^(10 - off)) in both halves (exact)
  const uint32_t e = 25u - off;
  return -as_f16x2((e << 10) | (e << 26));
}

// Decode the 8 codes of MFMA step `s` from a lane's 16-byte code block into
// the fp16 B fragment (values in the K order the packer laid out).
template <class F>
__device__ inline f16x8 dequant_step(const typename F::CodeT& c, const PBuf<F::EB>& pb, int s,
                                     const DeqConsts& k) {
  // parameter index inside the entry for lane-local codes [8s, 8s+8)
  const int p = F::kGroup < F::SPAN ? (8 * s) / F::kGroup : 0;
  f16x2 out[4];
  if constexpr (F::kFmt == MOE_W_ASYM) {
    const uint32_t sm = pb.w[p];
    const f16x2 s2 = as_f16x2((sm & 0xffffu) * 0x10001u);
    const f16x2 m2 = as_f16x2((sm >> 16) * 0x10001u);
    if constexpr (F::kBits == 4) {
      // word s: pairs at offsets 0, 4 (low byte) and 0, 4 after >> 8
      const uint32_t d = c[s];
      const uint32_t e = d >> 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t src = i < 2 ? d : e;
        const int j = i & 1;
        const uint32_t t = (src & k.mask[j]) | k.magic[j];
        out[i] = __builtin_elementwise_fma(as_f16x2(t) + magic_sub(4 * j), s2, m2);
      }
    } else if constexpr (F::kBits == 3) {
      // low two bits as in the 2-bit layout (word s/2, byte s & 1), the high
      // bit as in the 1-bit layout (word s/4, bits 4(s & 3)..)
      const uint32_t d = c.lo[s >> 1];
      const uint32_t lo = (s & 1) ? d >> 8 : d;
      const uint32_t hi = c.hi[s >> 2] >> (4 * (s & 3));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t tl = (lo & k.mask[j]) | k.magic[j];
        const uint32_t th = (hi & k.mask_h[j]) | k.magic_h[j];
        const f16x2 q = (as_f16x2(th) + magic3_sub(j)) + as_f16x2(tl);
        out[j] = __builtin_elementwise_fma(q, s2, m2);
      }
    } else if (F::kBits == 1) {
      // word s/4 holds four steps; step s uses bits 4q..4q+3 of each 16-bit
      // half, q = s & 3 (bits of the other half shifted in stay masked out)
      const uint32_t src = c[s >> 2] >> (4 * (s & 3));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = (src & k.mask[j]) | k.magic[j];
        out[j] = __builtin_elementwise_fma(as_f16x2(t) + magic_sub(j), s2, m2);
      }
    } else {
      // word s/2 holds two steps; step s uses offsets 0, 2, 4, 6 of byte (s & 1)
      const uint32_t d = c[s >> 1];
      const uint32_t src = (s & 1) ? d >> 8 : d;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t t = (src & k.mask[j]) | k.magic[j];
        out[j] = __builtin_elementwise_fma(as_f16x2(t) + magic_sub(2 * j), s2, m2);
      }
    }
  } else {
    // e2m1: natural nibble order; the gfx950 converter maps byte b of the word
    // to (low nibble, high nibble) exactly (scale 1.0), then one fp16 multiply
    const uint32_t sw = (pb.w[p >> 1] >> (16 * (p & 1))) & 0xffffu;
    const f16x2 s2 = as_f16x2(sw * 0x10001u);
    const uint32_t d = c[s];
    out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * s2;
    out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * s2;
    out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * s2;
    out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * s2;
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
