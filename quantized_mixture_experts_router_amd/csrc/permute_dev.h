// Stable counting-sort permutation of the T*k (token, slot) assignments by
// expert, giving contiguous per-expert row segments for the grouped GEMMs.
//
// The pages give the grouping only as "route each token to its top-k experts"
// (Baidu Cloud quantized-MoE article, expert routing section; "Sparse
// activation ... 2% activation", section 2.2); the segment order is this
// library's choice: ascending token inside each expert, which makes the
// permutation unique and reproducible run to run.
//
// One block of 16 waves (permute_block): wave w owns a contiguous chunk of
// assignments.
//  1. per-wave expert histograms (LDS);
//  2. counts, offsets and per-(wave, expert) bases by prefix sums;
//  3. each wave walks its chunk 64 assignments at a time; a lane's rank among
//     earlier lanes with the same expert comes from ballots over the expert
//     id bits, so equal experts keep their assignment order.
#pragma once

#include "common.h"

namespace moeq {
namespace pm {

constexpr int kWaves = 16;  // the permutation kernel's block
constexpr int kThreads = kWaves * 64;

// int32 words of dynamic LDS that permute_block<W> needs
__host__ __device__ inline int permute_smem_words(int W, int E) { return W * E + W * 64 + 1; }

// Stable counting sort of the R = T*k assignments by the W * 64 threads of
// the block. Returns (to every thread) the flag bits found: ids equal to
// MOE_ID_NAN raise MOE_FLAG_NAN_LOGIT, any other id outside [0,E)
// MOE_FLAG_BAD_EXPERT_ID; such assignments get inv = -1 and no row.
template <int W>
__device__ inline uint32_t permute_block(const int32_t* __restrict__ ids, int R, int k, int E,
                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                  int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                  int32_t* sm) {
  constexpr int NTH = W * 64;
  int32_t* base = sm;                       // [W][E]
  int32_t* scan = sm + W * E;          // [NTH] scan scratch
  uint32_t* s_flags = (uint32_t*)(scan + NTH);
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;

  if (tid == 0) *s_flags = 0u;
  for (int i = tid; i < W * E; i += NTH) base[i] = 0;
  __syncthreads();

  const int chunk = ((R + W - 1) / W + 63) / 64 * 64;
  const int c0 = wave * chunk;
  const int c1 = min(R, c0 + chunk);

  // 1. histograms (ids loaded kB per lane at a time, all in flight at once)
  constexpr int kB = 8;
  uint32_t bad = 0u;
  for (int a0 = c0; a0 < c1; a0 += 64 * kB) {
    int ev[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) ev[u] = ids[min(a0 + 64 * u + lane, c1 - 1)];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (a0 + 64 * u + lane >= c1) break;
      const int e = ev[u];
      if (e >= 0 && e < E)
        atomicAdd(&base[wave * E + e], 1);
      else
        bad |= e == MOE_ID_NAN ? (uint32_t)MOE_FLAG_NAN_LOGIT : (uint32_t)MOE_FLAG_BAD_EXPERT_ID;
    }
  }
  if (bad) atomicOr(s_flags, bad);
  __syncthreads();

  // 2. per-expert totals (thread e loops over waves), then exclusive scan
  const int EPT = (E + NTH - 1) / NTH;  // experts per thread (1 for E <= 1024)
  int local_total = 0;
  for (int q = 0; q < EPT; ++q) {
    int e = tid * EPT + q;
    if (e < E) {
      int run = 0;
      for (int w = 0; w < W; ++w) {
        int c = base[w * E + e];
        base[w * E + e] = run;
        run += c;
      }
      counts[e] = run;
      local_total += run;
    }
  }
  scan[tid] = local_total;
  __syncthreads();
  for (int off = 1; off < NTH; off <<= 1) {
    int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  int excl = scan[tid] - local_total;
  for (int q = 0; q < EPT; ++q) {
    int e = tid * EPT + q;
    if (e < E) {
      int c = 0;
      for (int w = 0; w < W; ++w) base[w * E + e] += excl;
      offsets[e] = excl;
      // counts[e] was written above; recompute the running prefix
      c = counts[e];
      excl += c;
    }
  }
  if (tid == NTH - 1) offsets[E] = scan[NTH - 1];
  __syncthreads();

  // 3. stable scatter
  const int bits = 32 - __clz(E > 1 ? E - 1 : 1);
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int p0 = c0; p0 < c1; p0 += 64 * kB) {
    int ev[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) ev[u] = ids[min(p0 + 64 * u + lane, c1 - 1)];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int p = p0 + 64 * u;
      if (p >= c1) break;  // uniform: p is the same in every lane
      const int a = p + lane;
      const int e = a < c1 ? ev[u] : -1;
      const bool valid = e >= 0 && e < E;
      uint64_t m = __ballot(valid);
      for (int b = 0; b < bits; ++b) {
        const uint64_t bb = __ballot(valid && ((e >> b) & 1));
        m &= ((e >> b) & 1) ? bb : ~bb;
      }
      if (valid) {
        const int rank = __popcll(m & lt_mask);
        const int pos = base[wave * E + e] + rank;
        perm[pos] = a / k;
        inv[a] = pos;
        const bool last = (m >> lane) == 1ull;  // no same-expert lane above this one
        if (last) base[wave * E + e] += rank + 1;
      } else if (a < c1) {
        inv[a] = -1;
      }
    }
  }
  __syncthreads();
  return *s_flags;
}

}  // namespace pm
}  // namespace moeq
