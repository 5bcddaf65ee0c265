// Router device code shared by the routing kernel and the fused small-batch
// front kernel: fp64 logits of a group of tokens, top-k and softmax.
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
// A group = TG x 2 tokens x all experts, computed by NT threads. Each thread
// owns a 2-token x 8-expert register tile and a slice of the hidden
// dimension: slices are 8 columns wide and interleaved, so neighbouring
// lanes read neighbouring 16-/32-byte chunks of the same rows. Partial sums
// meet through wavefront butterflies and LDS, then each wavefront runs the
// top-k of its tokens with wave-wide (value desc, index asc) argmax rounds.
#pragma once

#include "common.h"

namespace moeq {
namespace rt {

constexpr int kTM = 2;         // tokens per thread
constexpr int kEM = 8;         // experts per thread
constexpr int kInvalid = 0x7fffffff;

// Raw operands of one 8-column slice: x of kTM tokens (bf16 pairs or fp32)
// and Wr of kEM experts. Loaded for a whole batch of slices before any use,
// so that a thread waits for memory once per batch.
template <int XDT>
struct Slice {
  static constexpr int XW = XDT == MOE_BF16 ? 4 : 8;  // 32-bit words of x per token
  uint32_t x[kTM][XW];
  f32x4 w[kEM][2];
};

template <int XDT>
__device__ inline void load_slice(const void* x, const float* Wr, const int* trow, const int* erow,
                                  int H, int h, Slice<XDT>& o) {
#pragma unroll
  for (int i = 0; i < kTM; ++i) {
    if (XDT == MOE_BF16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)x + (size_t)trow[i] * H + h);
#pragma unroll
      for (int q = 0; q < 4; ++q) o.x[i][q] = v[q];
    } else {
      const u32x4* p = reinterpret_cast<const u32x4*>((const float*)x + (size_t)trow[i] * H + h);
      const u32x4 a = p[0], b = p[1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o.x[i][q] = a[q];
        o.x[i][4 + q] = b[q];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kEM; ++j) {
    const f32x4* wp = reinterpret_cast<const f32x4*>(Wr + (size_t)erow[j] * H + h);
    o.w[j][0] = wp[0];
    o.w[j][1] = wp[1];
  }
}

template <int XDT>
__device__ inline void fma_slice(const Slice<XDT>& o, double (&acc)[kTM][kEM]) {
  double xv[kTM][8];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (XDT == MOE_BF16) {
        xv[i][2 * q] = (double)__uint_as_float(o.x[i][q] << 16);
        xv[i][2 * q + 1] = (double)__uint_as_float(o.x[i][q] & 0xffff0000u);
      } else {
        xv[i][q] = (double)__uint_as_float(o.x[i][q]);
        xv[i][4 + q] = (double)__uint_as_float(o.x[i][4 + q]);
      }
    }
#pragma unroll
  for (int j = 0; j < kEM; ++j) {
    double wv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      wv[q] = (double)o.w[j][0][q];
      wv[4 + q] = (double)o.w[j][1][q];
    }
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][j] = fma(xv[i][q], wv[q], acc[i][j]);
  }
}

// hidden-dimension slices per (token group, expert group): the largest
// power of two with KS * TG * EG <= NT
__host__ __device__ inline int route_slices(int NT, int TG, int EG) {
  int ks = 1;
  while (2 * ks * TG * EG <= NT) ks *= 2;
  return ks;
}

// doubles of dynamic LDS that route_group needs
__host__ __device__ inline int route_smem_doubles(int NT, int TG, int E) {
  const int EG = (E + kEM - 1) / kEM;
  const int KS = route_slices(NT, TG, EG);
  const int NW = KS > 64 ? KS / 64 : 1;
  return (NW > 1 ? NW * TG * EG * kTM * kEM : 0) + TG * kTM * (E + 1);
}

// Logits, top-k ids and softmax weights of tokens [t0, t0 + 2 TG) (those
// below T), computed by the NT threads of the block. A token whose logits
// include a NaN gets MOE_ID_NAN in every slot and weight 0. Ends with the
// outputs written by the threads that own them (no trailing barrier).
template <int XDT, int NT>
__device__ void route_group(const void* __restrict__ x, const float* __restrict__ Wr,
                            const float* __restrict__ bias, int T, int H, int E, int k, int TG,
                            int t0, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                            float* __restrict__ logits_out, double* smem) {
  const int tid = threadIdx.x;
  const int TB = TG * kTM;
  const int EG = (E + kEM - 1) / kEM;             // expert groups
  const int KS = route_slices(NT, TG, EG);        // hidden-dimension slices
  const int active = KS * TG * EG;                // threads with work (<= NT)
  // lane -> (slice, token group, expert group); slice varies fastest
  const int ks = tid % KS;
  const int tg = (tid / KS) % TG;
  const int eg = tid / (KS * TG);
  const bool on = tid < active;

  double acc[kTM][kEM];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kEM; ++j) acc[i][j] = 0.0;

  if (on) {
    int trow[kTM];
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int t = t0 + tg * kTM + i;
      trow[i] = t < T ? t : 0;
    }
    int erow[kEM];
#pragma unroll
    for (int j = 0; j < kEM; ++j) erow[j] = min(eg * kEM + j, E - 1);
    // slices h = 8 ks + 8 KS i, i < ns, in pairs whose loads are all issued
    // before either slice is used; an odd last slice on its own
    const int ns = 8 * ks < H ? (H - 8 * ks + 8 * KS - 1) / (8 * KS) : 0;
    int i = 0;
    for (; i + 1 < ns; i += 2) {
      Slice<XDT> s0, s1;
      load_slice<XDT>(x, Wr, trow, erow, H, 8 * ks + 8 * KS * i, s0);
      load_slice<XDT>(x, Wr, trow, erow, H, 8 * ks + 8 * KS * (i + 1), s1);
      __builtin_amdgcn_sched_barrier(0);  // keep every load of the pair ahead of the FMAs
      fma_slice<XDT>(s0, acc);
      fma_slice<XDT>(s1, acc);
    }
    if (i < ns) {
      Slice<XDT> s0;
      load_slice<XDT>(x, Wr, trow, erow, H, 8 * ks + 8 * KS * i, s0);
      fma_slice<XDT>(s0, acc);
    }
  }

  // reduce the hidden slices. Slices of one (token group, expert group) are
  // adjacent lanes (KS is a power of two): butterfly within the wavefront,
  // then across wavefronts through LDS when KS > 64.
  const int KW = KS < 64 ? KS : 64;  // slices per wavefront
  if (KS > 1) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kEM; ++j)
        for (int off = 1; off < KW; off <<= 1) acc[i][j] += __shfl_xor(acc[i][j], off);
  }
  const int NW = KS / KW;  // wavefronts per (token group, expert group)
  double* part = smem;     // [group][i][j][NW]
  if (NW > 1 && on && (ks % KW) == 0) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kEM; ++j)
        part[(((size_t)(eg * TG + tg) * kTM + i) * kEM + j) * NW + ks / KW] = acc[i][j];
  }
  __syncthreads();
  double* lg = smem + (NW > 1 ? (size_t)NW * TG * EG * kTM * kEM : 0);  // [TB][E+1]
  if (NW > 1) {
    const int nslots = TG * EG * kTM * kEM;
    for (int slot = tid; slot < nslots; slot += NT) {
      double v = 0.0;
      for (int q = 0; q < NW; ++q) v += part[(size_t)slot * NW + q];
      const int j = slot % kEM, i = (slot / kEM) % kTM, g = slot / (kEM * kTM);
      const int tgi = g % TG, egi = g / TG;
      const int e = egi * kEM + j, tt = tgi * kTM + i;
      if (e < E) lg[tt * (E + 1) + e] = v;
    }
  } else if (on && ks == 0) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kEM; ++j) {
        const int e = eg * kEM + j;
        if (e < E) lg[(tg * kTM + i) * (E + 1) + e] = acc[i][j];
      }
  }
  __syncthreads();
  // bias; optional fp32 logits
  for (int i = tid; i < TB * E; i += NT) {
    const int tt = i / E, e = i % E;
    double v = lg[tt * (E + 1) + e] + (bias ? (double)bias[e] : 0.0);
    lg[tt * (E + 1) + e] = v;
    if (logits_out && t0 + tt < T) logits_out[(size_t)(t0 + tt) * E + e] = (float)v;
  }
  __syncthreads();

  // top-k: wavefront w handles tokens w, w + NT/64, ...
  const int wave = tid / 64, lane = tid % 64;
  const int EPL = (E + 63) / 64;  // candidates per lane (<= 4)
  for (int tt = wave; tt < TB; tt += NT / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    const double* row = lg + tt * (E + 1);
    uint32_t taken = 0;
    bool nan_seen = false;
    double my_v = 0.0, top_v = 0.0;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      double bv = 0.0;
      int bi = kInvalid;
      for (int j = 0; j < EPL; ++j) {
        int e = lane + 64 * j;
        if (e < E && !((taken >> j) & 1u)) {
          double v = row[e];
          if (v != v) nan_seen = true;
          if (bi == kInvalid || v > bv) {  // increasing e: ties keep the lower index
            bv = v;
            bi = e;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        double ov = __shfl_xor(bv, off);
        int oi = __shfl_xor(bi, off);
        bool better = oi != kInvalid && (bi == kInvalid || ov > bv || (ov == bv && oi < bi));
        if (better) {
          bv = ov;
          bi = oi;
        }
      }
      if (r == 0) top_v = bv;
      if (lane == r) {
        my_v = bv;
        my_i = bi;
      }
      if (bi != kInvalid && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    // a NaN anywhere in the row makes the whole routing of the token undefined
    const bool nan_row = __any(nan_seen);
    double ex = lane < k ? exp(my_v - top_v) : 0.0;
    double den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (lane < k) {
      ids_out[(size_t)t * k + lane] = nan_row ? MOE_ID_NAN : my_i;
      w_out[(size_t)t * k + lane] = nan_row ? 0.f : (float)(ex / den);
    }
  }
}

}  // namespace rt
}  // namespace moeq
