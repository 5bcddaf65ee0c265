// Router device code: fp64 logits on the matrix cores, and the per-token
// top-k + softmax that the routing kernel and the fused small-batch front
// kernel share.
//
// Method: Baidu Cloud article on quantized MoE LLM inference, "expert
// routing" section (router linear -> top-k -> softmax over the top-k ->
// weighted sum); "Sparse activation ... GPT-4's 2% activation", section 2.2
// (keep the K highest of E logits). The router stays unquantised (mixed-
// precision notes, section 2.1: int8 logits lose the small gaps between
// experts), so logits are accumulated in fp64: products of bf16/fp32 inputs
// with fp32 weights are exact in fp64 and the sum carries ~1e-16 relative
// error, far below the 1e-6 gap at which a token counts as a near-tie.
//
// Logits. gfx950's fp64 matrix instruction (16x16x4, D = A B + C) runs the
// contraction. A wavefront owns 16 tokens x NTW*16 experts over a range of
// hidden-dimension chunks of 16 columns. In a chunk, lane (r = lane % 16,
// g = lane / 16) loads columns [4g, 4g+4) of token row r and of expert row r
// of each 16-expert tile; step s of the chunk then feeds column 4g + s as
// k-index g of A (token r) and B (expert r). Any bijection between (step,
// k-index) and columns gives the same dot products, and this one makes every
// lane's loads contiguous 8/16-byte reads. Output: element i of lane l is
// D[4i + l/16][l%16] (token 4i + g, expert r). The waves of a block split
// the hidden dimension and add their tiles in LDS in wave order; blocks that
// split it further leave fp64 partial logits that the top-k adds in block
// order. Every sum is in a fixed order, so results do not depend on
// scheduling.
#pragma once

#include "common.h"

namespace moeq {
namespace rt {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kTT = 16;  // tokens per wavefront tile

// raw operands of one 16-column chunk for one lane: a token row, NTW
// expert rows
template <int XDT, int NTW>
struct Chunk {
  static constexpr int XW = XDT == MOE_BF16 ? 2 : 4;  // 32-bit words of x (4 columns)
  uint32_t x[XW];
  f32x4 w[NTW];
};

template <int XDT, int NTW>
__device__ inline void load_chunk(const void* x, const float* Wr, size_t xoff,
                                  const size_t (&woff)[NTW], int col, Chunk<XDT, NTW>& o) {
  if (XDT == MOE_BF16) {
    const u32x2 v = *reinterpret_cast<const u32x2*>((const uint16_t*)x + xoff + col);
    o.x[0] = v[0];
    o.x[1] = v[1];
  } else {
    const u32x4 v = *reinterpret_cast<const u32x4*>((const float*)x + xoff + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) o.x[q] = v[q];
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j) o.w[j] = *reinterpret_cast<const f32x4*>(Wr + woff[j] + col);
}

template <int XDT>
__device__ inline float x_val(const uint32_t* xw, int s) {
  if (XDT == MOE_BF16) return __uint_as_float(s & 1 ? (xw[s >> 1] & 0xffff0000u) : (xw[s >> 1] << 16));
  return __uint_as_float(xw[s]);
}

// the four k-steps of one chunk; CHECK: zero the operands of a lane whose
// columns lie past the row end (or of a chunk past the range)
template <int XDT, int NTW, bool CHECK>
__device__ inline void mma_chunk(const Chunk<XDT, NTW>& c, bool valid, f64x4 (&acc)[NTW]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    double a = (double)x_val<XDT>(c.x, s);
    if (CHECK && !valid) a = 0.0;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      double b = (double)c.w[j][s];
      if (CHECK && !valid) b = 0.0;
      acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[j], 0, 0, 0);
    }
  }
}

// Adds to acc the products of tokens [t0, t0 + 16) x experts
// [e0, e0 + 16 NTW) over the chunks [c0, c1) (c0 < c1); rows past T or E
// repeat the last row (their sums are never stored).
template <int XDT, int NTW>
__device__ inline void logits_acc(const void* __restrict__ x, const float* __restrict__ Wr, int T,
                                  int H, int E, int t0, int e0, int c0, int c1,
                                  f64x4 (&acc)[NTW]) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const size_t xoff = (size_t)min(t0 + r, T - 1) * H + 4 * g;
  size_t woff[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) woff[j] = (size_t)min(e0 + 16 * j + r, E - 1) * H + 4 * g;
  // A lane's columns 16c + 4g + [0,4) lie inside the row iff 16c + 4g < H
  // (H is a multiple of 8): every chunk below H / 16 is whole. Pairs of
  // whole chunks run without checks, two in flight (the loads of the next
  // go out before the current one is multiplied); what is left (a half
  // chunk, an odd chunk) runs with them.
  auto col_of = [&](int c) { return min(16 * min(c, c1 - 1), H - 4 - 4 * g); };
  const int cw = min(c1, H / 16);  // end of the whole chunks
  Chunk<XDT, NTW> ca, cb;
  load_chunk<XDT, NTW>(x, Wr, xoff, woff, col_of(c0), ca);
  int c = c0;
  for (; c + 1 < cw; c += 2) {
    load_chunk<XDT, NTW>(x, Wr, xoff, woff, col_of(c + 1), cb);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the multiplies
    mma_chunk<XDT, NTW, false>(ca, true, acc);
    __builtin_amdgcn_sched_barrier(0);
    load_chunk<XDT, NTW>(x, Wr, xoff, woff, col_of(c + 2), ca);
    __builtin_amdgcn_sched_barrier(0);
    mma_chunk<XDT, NTW, false>(cb, true, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ca holds chunk c (clamped) here
  for (; c < c1; ++c) {
    mma_chunk<XDT, NTW, true>(ca, 16 * c + 4 * g < H, acc);
    if (c + 1 < c1) load_chunk<XDT, NTW>(x, Wr, xoff, woff, col_of(c + 1), ca);
  }
}

// Order key of a candidate: the fp64 value's bits made monotone as an
// unsigned integer, the low 8 bits replaced by 255 - e so that the maximum
// key is the largest value and, among equal values, the lowest expert index.
// Keys drop 8 of the 52 mantissa bits, so two values within ~2^-44 of each
// other (relative) may be ordered by index rather than by value; such a pair
// is a near-tie by orders of magnitude (gap < 1e-6) and never decides an id
// that is compared exactly.
__device__ inline uint64_t order_key(double v, int e) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u = (u >> 63) ? ~u : (u | (1ull << 63));
  return (u & ~0xFFull) | (uint64_t)(255 - e);
}

template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of a key over the 64 lanes, returned to every lane (all lanes
// active): DPP swaps within each 16-lane row (lane ^ 1, lane ^ 2, rotate by
// 4 and 8), then lane ^ 16 and lane ^ 32.
__device__ inline uint64_t wave_max_u64(uint64_t k) {
  k = umax64(k, dpp_u64<0xB1>(k));   // quad_perm [1,0,3,2]
  k = umax64(k, dpp_u64<0x4E>(k));   // quad_perm [2,3,0,1]
  k = umax64(k, dpp_u64<0x124>(k));  // row_ror:4
  k = umax64(k, dpp_u64<0x128>(k));  // row_ror:8
  k = umax64(k, (uint64_t)__shfl_xor((unsigned long long)k, 16));
  k = umax64(k, (uint64_t)__shfl_xor((unsigned long long)k, 32));
  return k;
}

// Routing of token t by one wavefront (all 64 lanes active): lane l holds
// the logits of experts l, l + 64, l + 128, l + 192 (those below E), each
// the KB partial sums P[kb][t][e] added in kb order plus the bias, all
// loaded up front. Then k rounds of a wave-wide argmax over the untaken
// candidates; the softmax over the k winners' exact fp64 logits. A NaN
// among the token's logits makes its routing undefined: every slot gets
// MOE_ID_NAN and weight 0. logits_out (optional) receives the fp32 logits;
// ids_lds (optional, LDS) a copy of the ids.
// Token t's logits L[t, lane + 64 j] (j < 4, clamped to E-1 past E) into
// cand[]: the KB fp64 partials added in kb order, then the bias.
__device__ inline void token_logits(const double* __restrict__ P, int KB,
                                    const float* __restrict__ bias, int T, int E, int t,
                                    int ec[4], double cand[4]) {
  const int lane = threadIdx.x & 63;
  const size_t stride = (size_t)T * E;
  const double* row = P + (size_t)t * E;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ec[j] = min(lane + 64 * j, E - 1);
    cand[j] = 0.0;
  }
  // partials in batches of 4 (16 loads in flight), added in kb order
  for (int q0 = 0; q0 < KB; q0 += 4) {
    double pv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[u][j] = row[(size_t)min(q0 + u, KB - 1) * stride + ec[j]];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (q0 + u < KB) cand[j] += pv[u][j];
  }
  if (bias) {
#pragma unroll
    for (int j = 0; j < 4; ++j) cand[j] += (double)bias[ec[j]];
  }
}

// qscale/qzero (optional, per expert; the int8 router logits of the AlphaQ
// blog's DRAQ, section 4.1): the router ranks and weighs the logits after an
// affine int8 round trip, (clamp(rint(L/s) + z, -128, 127) - z) * s, in
// fp64; experts with s <= 0 (or NaN) get 0. NaN detection and logits_out use
// the logits before it.
__device__ inline void topk_token(const double* __restrict__ P, int KB, const float* __restrict__ bias,
                                  int T, int E, int k, int t, int32_t* __restrict__ ids_out,
                                  float* __restrict__ w_out, float* __restrict__ logits_out,
                                  int32_t* ids_lds = nullptr, const float* __restrict__ qscale = nullptr,
                                  const int32_t* __restrict__ qzero = nullptr) {
  const int lane = threadIdx.x & 63;
  int ec[4];
  double cand[4];
  token_logits(P, KB, bias, T, E, t, ec, cand);
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      nan_seen |= cand[j] != cand[j];
      if (logits_out) logits_out[(size_t)t * E + e] = (float)cand[j];
    }
    if (qscale) {
      const double sc = (double)qscale[ec[j]];
      const double z = (double)qzero[ec[j]];
      double q = rint(cand[j] / sc) + z;
      q = q < -128.0 ? -128.0 : (q > 127.0 ? 127.0 : q);
      cand[j] = sc > 0.0 ? (q - z) * sc : 0.0;
    }
  }
  uint32_t taken = 0;
  double my_v = 0.0, top_v = 0.0;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
    double best_v = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      const uint64_t key = (e < E && !((taken >> j) & 1u)) ? order_key(cand[j], e) : 0ull;
      if (key > best) {
        best = key;
        best_v = cand[j];
      }
    }
    const uint64_t win = wave_max_u64(best);
    const int wi = 255 - (int)(win & 0xFF);
    const double wv = __shfl(best_v, wi & 63);  // the owner's exact logit
    if (r == 0) top_v = wv;
    if (lane == r) {
      my_v = wv;
      my_i = wi;
    }
    if ((wi & 63) == lane) taken |= 1u << (wi >> 6);
  }
  const bool nan_row = __any(nan_seen);
  const double ex = lane < k ? exp(my_v - top_v) : 0.0;
  double den = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if (lane < k) {
    const int id = nan_row ? MOE_ID_NAN : my_i;
    ids_out[(size_t)t * k + lane] = id;
    w_out[(size_t)t * k + lane] = nan_row ? 0.f : (float)(ex / den);
    if (ids_lds) ids_lds[t * k + lane] = id;  // a copy for a consumer in the same block
  }
}

}  // namespace rt
}  // namespace moeq
