// Permutation kernel: one block runs permute_block (permute_dev.h) and
// stores the flag word of the call.
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

}  // namespace

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts,
                          int32_t* offsets, int32_t* perm, int32_t* inv, uint32_t* flags,
                          hipStream_t s) {
  const int R = T * k;
  const size_t smem = sizeof(int32_t) * pm::permute_smem_words(pm::kWaves, E);
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(pm::kThreads), smem, s, ids, R, k, E, counts,
                     offsets, perm, inv, flags);
  return hipGetLastError();
}

}  // namespace moeq
