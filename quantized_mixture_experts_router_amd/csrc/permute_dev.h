// Stable counting-sort permutation of the T*k (token, slot) assignments by
// expert, giving contiguous per-expert row segments for the grouped GEMMs.
//
// The pages give the grouping only as "route each token to its top-k experts"
// (Baidu Cloud quantized-MoE article, expert routing section; "Sparse
// activation ... 2% activation", section 2.2); the segment order is this
// library's choice: ascending token inside each expert, which makes the
// permutation unique and reproducible run to run.
//
// Building blocks, each run by one wavefront over a contiguous slice of
// assignments (ids loaded kB per lane at a time, all in flight at once):
//  - wave_hist: per-expert counts of the slice into an LDS histogram;
//  - wave_scatter: walks the slice 64 assignments at a time; a lane's rank
//    among earlier lanes with the same expert comes from ballots over the
//    expert id bits, so equal experts keep their assignment order, and the
//    per-expert running bases (LDS) advance by the counts.
// permute_block sorts everything with one block; the multi-block kernels in
// permute.hip split the assignments over blocks with the same pieces.
#pragma once

#include "common.h"

namespace moeq {
namespace pm {

constexpr int kWaves = 16;  // the single-block permutation kernel's block
constexpr int kThreads = kWaves * 64;
constexpr int kB = 8;       // ids per lane in flight

// flag bits of an id outside [0, E)
__device__ inline uint32_t bad_bits(int e) {
  return e == MOE_ID_NAN ? (uint32_t)MOE_FLAG_NAN_LOGIT : (uint32_t)MOE_FLAG_BAD_EXPERT_ID;
}

// Adds the expert counts of assignments [c0, c1) to hist[E] (LDS); returns
// (per lane) the flag bits of the ids outside [0, E).
__device__ inline uint32_t wave_hist(const int32_t* __restrict__ ids, int c0, int c1, int E,
                                     int32_t* hist) {
  const int lane = threadIdx.x & 63;
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
        atomicAdd(&hist[e], 1);
      else
        bad |= bad_bits(e);
    }
  }
  return bad;
}

// Stable scatter of assignments [c0, c1): row base[e] + rank for the r-th
// assignment of expert e in the slice (base[] in LDS, advanced as it goes).
// Assignment a belongs to token a / k. Ids outside [0, E) get inv = -1.
// perm_lds (optional, LDS) receives a copy of the perm entries written.
__device__ inline void wave_scatter(const int32_t* __restrict__ ids, int c0, int c1, int E, int k,
                                    int32_t* base, int32_t* __restrict__ perm,
                                    int32_t* __restrict__ inv, int32_t* perm_lds = nullptr) {
  const int lane = threadIdx.x & 63;
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
        const int pos = base[e] + rank;
        perm[pos] = a / k;
        if (perm_lds) perm_lds[pos] = a / k;
        inv[a] = pos;
        const bool last = (m >> lane) == 1ull;  // no same-expert lane above this one
        if (last) base[e] += rank + 1;
      } else if (a < c1) {
        inv[a] = -1;
      }
    }
  }
}

// In-block exclusive scan of one int per thread (NTH threads, scan[NTH] in
// LDS); returns the thread's exclusive prefix, and the total in *total.
template <int NTH>
__device__ inline int block_excl_scan(int v, int* scan, int* total) {
  const int tid = threadIdx.x;
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < NTH; off <<= 1) {
    const int o = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += o;
    __syncthreads();
  }
  const int incl = scan[tid];
  *total = scan[NTH - 1];
  __syncthreads();
  return incl - v;
}

// int32 words of dynamic LDS that permute_block<W> needs
__host__ __device__ inline int permute_smem_words(int W, int E) { return W * E + W * 64 + 1; }

// Stable counting sort of the R = T*k assignments by the W * 64 threads of
// the block. Returns (to every thread) the flag bits found: ids equal to
// MOE_ID_NAN raise MOE_FLAG_NAN_LOGIT, any other id outside [0,E)
// MOE_FLAG_BAD_EXPERT_ID; such assignments get inv = -1 and no row.
// Optional LDS copies for a consumer in the same block: perm_lds[R] of
// perm, *rows_lds of offsets[E] (the rows written).
template <int W>
__device__ inline uint32_t permute_block(const int32_t* __restrict__ ids, int R, int k, int E,
                                         int32_t* __restrict__ counts,
                                         int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                         int32_t* __restrict__ inv, int32_t* sm,
                                         int32_t* perm_lds = nullptr, int32_t* rows_lds = nullptr) {
  constexpr int NTH = W * 64;
  int32_t* base = sm;              // [W][E]
  int32_t* scan = sm + W * E;      // [NTH] scan scratch
  uint32_t* s_flags = (uint32_t*)(scan + NTH);
  const int tid = threadIdx.x;
  const int wave = tid / 64;

  if (tid == 0) *s_flags = 0u;
  for (int i = tid; i < W * E; i += NTH) base[i] = 0;
  __syncthreads();

  const int chunk = ((R + W - 1) / W + 63) / 64 * 64;
  const int c0 = wave * chunk;
  const int c1 = min(R, c0 + chunk);

  // 1. per-wave histograms
  const uint32_t bad = wave_hist(ids, c0, c1, E, base + wave * E);
  if (bad) atomicOr(s_flags, bad);
  __syncthreads();

  // 2. per-expert totals and the exclusive scan over experts, by wavefront 0
  //    alone (E <= 256: experts 4 lane .. 4 lane + 3 per lane, a shuffle scan
  //    over lanes), so the block waits at one barrier instead of a block
  //    scan's log2(NTH) pairs; the wave bases become prefixes over the waves
  if (wave == 0) {
    const int lane = tid & 63;
    int tot[4];
    int lane_sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      int run = 0;
      if (e < E) {
        for (int w = 0; w < W; ++w) {
          const int c = base[w * E + e];
          base[w * E + e] = run;
          run += c;
        }
      }
      tot[j] = run;
      lane_sum += run;
    }
    int incl = lane_sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int excl = incl - lane_sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) {
        for (int w = 0; w < W; ++w) base[w * E + e] += excl;
        counts[e] = tot[j];
        offsets[e] = excl;
      }
      excl += tot[j];
    }
    if (lane == 63) {
      offsets[E] = incl;
      if (rows_lds) *rows_lds = incl;
    }
  }
  __syncthreads();

  // 3. stable scatter
  wave_scatter(ids, c0, c1, E, k, base + wave * E, perm, inv, perm_lds);
  __syncthreads();
  return *s_flags;
}

}  // namespace pm
}  // namespace moeq
