// Router kernel: logits + top-k + softmax over the selected logits for
// blocks of 2..16 tokens (the arithmetic lives in route_dev.h).
#include "route_dev.h"

namespace moeq {

namespace {

constexpr int kThreads = 256;

// Token groups per block (2 tokens each): as few as keep the grid near 1024
// blocks (small batches spread the hidden dimension over every thread), but
// enough that re-reading the router weights per block stays under ~256 MB of
// L2 traffic (large E*H), and at most 8 (kTG * expert groups <= 256 threads).
__host__ __device__ inline int route_tgroups(int T, int H, int E) {
  int tg = 1;
  while (tg < 8 && (T + 2 * tg - 1) / (2 * tg) > 1024) tg *= 2;
  const double traffic = 2.0 * T * E * H;  // bytes of Wr reads with one group
  while (tg < 8 && traffic / tg > 256e6) tg *= 2;
  const int EG = (E + 7) / 8;
  while (tg > 1 && tg * EG > 256) tg /= 2;
  return tg;
}


template <int XDT>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias,
    int T, int H, int E, int k, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    float* __restrict__ logits_out) {
  extern __shared__ double smem[];
  const int TG = route_tgroups(T, H, E);
  rt::route_group<XDT, kThreads>(x, Wr, bias, T, H, E, k, TG, blockIdx.x * TG * rt::kTM, ids_out,
                                 w_out, logits_out, smem);
}

}  // namespace

hipError_t launch_route(const void* x, int xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int TG = route_tgroups(T, H, E), TB = TG * rt::kTM;
  const size_t smem = sizeof(double) * rt::route_smem_doubles(kThreads, TG, E);
  dim3 grid((T + TB - 1) / TB);
  if (xdt == MOE_BF16)
    hipLaunchKernelGGL(route_kernel<MOE_BF16>, grid, dim3(kThreads), smem, s, x, Wr, b, T, H, E, k,
                       ids, w, logits);
  else
    hipLaunchKernelGGL(route_kernel<MOE_F32>, grid, dim3(kThreads), smem, s, x, Wr, b, T, H, E, k,
                       ids, w, logits);
  return hipGetLastError();
}

}  // namespace moeq
