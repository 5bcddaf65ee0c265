// Permutation kernels (the sort itself is in permute_dev.h).
//  - Up to kPermuteSingleMax assignments: one block runs permute_block.
//  - Above: three launches over blocks of kMBWaves wavefronts, each block
//    owning a contiguous chunk of assignments:
//      1. permute_hist_kernel: per-block expert counts -> ghist[b][e];
//      2. permute_scan_kernel (one block): counts, offsets, and ghist[b][e]
//         turned into the block's first row of expert e (a prefix over
//         blocks, plus offsets[e]); the flag word;
//      3. permute_scatter_kernel: per-wave counts again, prefixes over the
//         block's waves, then the stable ballot scatter.
//    Blocks own ascending chunks and waves ascending slices of them, so the
//    result is the same stable order as the single-block sort.
#include "permute_dev.h"

namespace moeq {

namespace {

__global__ __launch_bounds__(pm::kThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv,
    uint32_t* __restrict__ flags) {
  extern __shared__ int32_t sm[];
  const uint32_t bits = pm::permute_block<pm::kWaves>(ids, R, k, E, counts, offsets, perm, inv, sm);
  if (threadIdx.x == 0 && flags) *flags = bits;  // the call's flag word starts here
}

constexpr int kMBWaves = 4;
constexpr int kMBThreads = kMBWaves * 64;

// slice of block b's wave w when blocks own chunks of CH assignments
__device__ inline void mb_slice(int R, int CH, int b, int w, int* c0, int* c1) {
  const int sl = CH / kMBWaves;
  *c0 = min(R, b * CH + w * sl);
  *c1 = min(R, *c0 + sl);
}

__global__ __launch_bounds__(kMBThreads) void permute_hist_kernel(
    const int32_t* __restrict__ ids, int R, int E, int CH, int32_t* __restrict__ ghist,
    uint32_t* __restrict__ gbits) {
  extern __shared__ int32_t sm[];  // hist[E], bits
  uint32_t* sbits = (uint32_t*)(sm + E);
  for (int i = threadIdx.x; i < E; i += kMBThreads) sm[i] = 0;
  if (threadIdx.x == 0) *sbits = 0u;
  __syncthreads();
  int c0, c1;
  mb_slice(R, CH, blockIdx.x, threadIdx.x / 64, &c0, &c1);
  const uint32_t bad = pm::wave_hist(ids, c0, c1, E, sm);
  if (bad) atomicOr(sbits, bad);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kMBThreads) ghist[(size_t)blockIdx.x * E + i] = sm[i];
  if (threadIdx.x == 0) gbits[blockIdx.x] = *sbits;
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(
    int B, int E, int32_t* __restrict__ ghist, const uint32_t* __restrict__ gbits,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, uint32_t* __restrict__ flags) {
  __shared__ int scan[kScanThreads];
  __shared__ uint32_t sbits;
  const int tid = threadIdx.x;
  if (tid == 0) sbits = 0u;
  __syncthreads();
  uint32_t bits = 0u;
  for (int b = tid; b < B; b += kScanThreads) bits |= gbits[b];
  if (bits) atomicOr(&sbits, bits);
  // per-expert prefix over blocks (8 loads in flight per step)
  const int EPT = (E + kScanThreads - 1) / kScanThreads;
  int local_total = 0;
  for (int q = 0; q < EPT; ++q) {
    const int e = tid * EPT + q;
    if (e < E) {
      int run = 0;
      for (int b0 = 0; b0 < B; b0 += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = ghist[(size_t)min(b0 + u, B - 1) * E + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (b0 + u < B) {
            ghist[(size_t)(b0 + u) * E + e] = run;
            run += c[u];
          }
        }
      }
      counts[e] = run;
      local_total += run;
    }
  }
  int total;
  int excl = pm::block_excl_scan<kScanThreads>(local_total, scan, &total);
  for (int q = 0; q < EPT; ++q) {
    const int e = tid * EPT + q;
    if (e < E) {
      offsets[e] = excl;
      excl += counts[e];
    }
  }
  if (tid == 0) {
    offsets[E] = total;
    *flags = sbits;  // the call's flag word starts here
  }
}

__global__ __launch_bounds__(kMBThreads) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int CH,
    const int32_t* __restrict__ ghist, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ int32_t sm[];  // [kMBWaves][E]
  for (int i = threadIdx.x; i < kMBWaves * E; i += kMBThreads) sm[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x / 64;
  int c0, c1;
  mb_slice(R, CH, blockIdx.x, wave, &c0, &c1);
  pm::wave_hist(ids, c0, c1, E, sm + wave * E);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kMBThreads) {
    int run = offsets[e] + ghist[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < kMBWaves; ++w) {
      const int c = sm[w * E + e];
      sm[w * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  pm::wave_scatter(ids, c0, c1, E, k, sm + wave * E, perm, inv);
}

}  // namespace

PermutePlan permute_plan(int R, int E) {
  PermutePlan p;
  p.blocks = 0;
  p.chunk = 0;
  p.scratch_bytes = 0;
  if (R <= kPermuteSingleMax) return p;
  // chunks of 2048 assignments (512 per wave), larger when that would take
  // more than 1024 blocks
  const long unit = 2048;
  long ch = unit * (((long)R + unit * 1024 - 1) / (unit * 1024));
  p.chunk = (int)ch;
  p.blocks = (int)(((long)R + ch - 1) / ch);
  p.scratch_bytes = align256((size_t)p.blocks * E * 4) + align256((size_t)p.blocks * 4);
  return p;
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, uint32_t* flags,
                          void* scratch, hipStream_t s) {
  const int R = T * k;
  const PermutePlan p = permute_plan(R, E);
  if (p.blocks == 0) {
    const size_t smem = sizeof(int32_t) * pm::permute_smem_words(pm::kWaves, E);
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(pm::kThreads), smem, s, ids, R, k, E, counts,
                       offsets, perm, inv, flags);
    return hipGetLastError();
  }
  // scratch: ghist [blocks][E], gbits [blocks]
  int32_t* ghist = (int32_t*)scratch;
  uint32_t* gbits = (uint32_t*)((char*)ghist + align256((size_t)p.blocks * E * 4));
  hipLaunchKernelGGL(permute_hist_kernel, dim3(p.blocks), dim3(kMBThreads),
                     sizeof(int32_t) * (E + 1), s, ids, R, E, p.chunk, ghist, gbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, p.blocks, E, ghist,
                     gbits, counts, offsets, flags);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(p.blocks), dim3(kMBThreads),
                     sizeof(int32_t) * kMBWaves * E, s, ids, R, k, E, p.chunk, ghist, offsets,
                     perm, inv);
  return hipGetLastError();
}

}  // namespace moeq
