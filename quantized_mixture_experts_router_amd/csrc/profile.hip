// Routing profile and precision tiers for expert-aware quantisation.
//
// The expert-aware quantisation digest (profiling and results sections)
// profiles which experts a task's tokens are routed to, keeps the most used
// ones ("hot") at higher precision and squeezes the rest to 2 bits; its
// conclusion sketches a gradient of ever coarser tiers as the experts get
// colder. Two pieces here:
//  - expert_hist_kernel: per-expert routing counts of a batch, added into an
//    int64 profile on the device (so a calibration run needs no host sync);
//  - plan_tiers: the host-side rule that turns a profile and a byte budget
//    into a tier per expert. Ranking by count (ties to the lower index),
//    each expert in turn takes the most precise tier that still leaves room
//    for all experts after it at the cheapest tier. This is the plainest
//    reading of "hottest most precise, as far as the budget allows": the
//    resulting tier vector, read in rank order, is the most precise one
//    (lexicographically) among all within the budget.
#include "profile.h"

#include <algorithm>
#include <numeric>
#include <vector>

namespace moeq {

namespace {

constexpr int kHistThreads = 256;
constexpr int kHistMaxE = 256;
constexpr int kHistU = 16;  // ids per thread loaded before their counts are added

__global__ __launch_bounds__(kHistThreads) void expert_hist_kernel(const int32_t* __restrict__ ids,
                                                                   long n, int E,
                                                                   unsigned long long* hist) {
  __shared__ unsigned int sh[kHistMaxE];
  for (int i = threadIdx.x; i < E; i += kHistThreads) sh[i] = 0u;
  __syncthreads();
  const long stride = (long)gridDim.x * kHistThreads;
  for (long a0 = (long)blockIdx.x * kHistThreads + threadIdx.x; a0 < n; a0 += stride * kHistU) {
    int e[kHistU];
#pragma unroll
    for (int u = 0; u < kHistU; ++u) {
      const long a = a0 + u * stride;
      e[u] = a < n ? ids[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kHistU; ++u)
      if (e[u] >= 0 && e[u] < E) atomicAdd(&sh[e[u]], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kHistThreads)
    if (sh[i]) atomicAdd(&hist[i], (unsigned long long)sh[i]);
}

}  // namespace

hipError_t launch_expert_histogram(const int32_t* ids, long n, int E, int64_t* hist,
                                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  // one pass of kHistU ids per thread where the grid allows (at most 1024
  // blocks; each adds its E counts into the E global words once)
  long blocks = (n + (long)kHistU * kHistThreads - 1) / ((long)kHistU * kHistThreads);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(expert_hist_kernel, dim3((unsigned)blocks), dim3(kHistThreads), 0, s, ids, n,
                     E, reinterpret_cast<unsigned long long*>(hist));
  return hipGetLastError();
}

bool plan_tiers(const int64_t* counts, int E, const uint64_t* tier_bytes, int ntiers,
                uint64_t budget, int32_t* tier_of, uint64_t* used_out) {
  const uint64_t last = tier_bytes[ntiers - 1];
  if ((uint64_t)E * last > budget) return false;
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return counts[a] > counts[b]; });
  std::vector<int32_t> tiers(E);
  uint64_t used = 0;
  for (int i = 0; i < E; ++i) {
    const uint64_t rest = (uint64_t)(E - 1 - i) * last;
    int t = ntiers - 1;
    for (int c = 0; c < ntiers; ++c) {
      if (used + tier_bytes[c] + rest <= budget) {
        t = c;
        break;
      }
    }
    tiers[order[i]] = t;
    used += tier_bytes[t];
  }
  std::copy(tiers.begin(), tiers.end(), tier_of);
  if (used_out) *used_out = used;
  return true;
}

}  // namespace moeq
