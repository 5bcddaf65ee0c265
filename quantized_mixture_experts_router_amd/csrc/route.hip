// Routing kernels: fp64 logits on the matrix cores (one block per 16-token
// tile x expert group, its wavefronts splitting the hidden dimension), then
// top-k + softmax with one wavefront per token. The arithmetic lives in
// route_dev.h; the split plan (route_plan) in common.h.
#include "profile.h"
#include "route_dev.h"

namespace moeq {

namespace {

// Block = KS wavefronts over one (token tile, expert group, K block). Wave
// ks accumulates chunks [c0 + ks*CPW, ...) of the block's K range; the KS
// partial tiles meet in LDS and are added in wave order, and the block
// stores the sum for its K block kb at P[kb][t][e].
template <int XDT, int NTW>
__global__ __launch_bounds__(1024) void route_logits_kernel(const void* __restrict__ x,
                                                            const float* __restrict__ Wr, int T,
                                                            int H, int E, int EG, int KS, int CPW,
                                                            double* __restrict__ P) {
  extern __shared__ double red[];  // [KS][NTW][4][64]
  const int TT = (T + rt::kTT - 1) / rt::kTT;
  const int NC = (H + 15) / 16;
  const int eg = blockIdx.x % EG;
  const int tt = (blockIdx.x / EG) % TT;
  const int kb = blockIdx.x / (EG * TT);
  const int ks = threadIdx.x / 64, lane = threadIdx.x & 63;
  const int t0 = tt * rt::kTT, e0 = eg * NTW * 16;
  const int c0 = (kb * KS + ks) * CPW, c1 = min(c0 + CPW, NC);
  rt::f64x4 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) acc[j] = rt::f64x4{0.0, 0.0, 0.0, 0.0};
  if (c0 < c1) rt::logits_acc<XDT, NTW>(x, Wr, T, H, E, t0, e0, c0, c1, acc);
  double* out = P + (size_t)kb * T * E;
  if (KS == 1) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * i + (lane >> 4), e = e0 + 16 * j + (lane & 15);
        if (t < T && e < E) out[(size_t)t * E + e] = acc[j][i];
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((ks * NTW + j) * 4 + i) * 64 + lane] = acc[j][i];
  __syncthreads();
  for (int v = threadIdx.x; v < NTW * 4 * 64; v += KS * 64) {
    const int l = v & 63, i = (v >> 6) & 3, j = v >> 8;
    const int t = t0 + 4 * i + (l >> 4), e = e0 + 16 * j + (l & 15);
    double sum = 0.0;
    for (int q = 0; q < KS; ++q) sum += red[((q * NTW + j) * 4 + i) * 64 + l];
    if (t < T && e < E) out[(size_t)t * E + e] = sum;
  }
}

// Top-k + softmax, one wavefront per token.
constexpr int kTopkThreads = 256;

__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const double* __restrict__ P, int KB, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ logits) {
  const int t = blockIdx.x * (kTopkThreads / 64) + threadIdx.x / 64;
  if (t < T) rt::topk_token(P, KB, bias, T, E, k, t, ids, w, logits);
}

// The same with the int8 round trip of the logits (qscale/qzero per expert).
__global__ __launch_bounds__(kTopkThreads) void route_topk_q_kernel(
    const double* __restrict__ P, int KB, const float* __restrict__ bias, int T, int E, int k,
    const float* __restrict__ qscale, const int32_t* __restrict__ qzero,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ logits) {
  const int t = blockIdx.x * (kTopkThreads / 64) + threadIdx.x / 64;
  if (t < T) rt::topk_token(P, KB, bias, T, E, k, t, ids, w, logits, nullptr, qscale, qzero);
}

// fp64 min / max through compare-and-swap on the 64-bit word
__device__ inline void atomic_min_f64(double* addr, double v) {
  unsigned long long* a = reinterpret_cast<unsigned long long*>(addr);
  unsigned long long old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (__longlong_as_double((long long)old) > v) {
    const unsigned long long got = atomicCAS(a, old, (unsigned long long)__double_as_longlong(v));
    if (got == old) break;
    old = got;
  }
}
__device__ inline void atomic_max_f64(double* addr, double v) {
  unsigned long long* a = reinterpret_cast<unsigned long long*>(addr);
  unsigned long long old = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  while (__longlong_as_double((long long)old) < v) {
    const unsigned long long got = atomicCAS(a, old, (unsigned long long)__double_as_longlong(v));
    if (got == old) break;
    old = got;
  }
}

constexpr int kRangeWaves = 4;

// Calibration of the int8 router logits: the smallest and largest fp64 logit
// of every expert over the tokens, merged into lo[E] / hi[E] (NaN logits
// skipped). A wavefront walks tokens (lane + 64 j = expert), the block's
// wavefronts meet in LDS, then one compare-and-swap per expert and block.
__global__ __launch_bounds__(64 * kRangeWaves) void logit_range_kernel(
    const double* __restrict__ P, int KB, const float* __restrict__ bias, int T, int E,
    double* __restrict__ lo, double* __restrict__ hi) {
  __shared__ double smin[kRangeWaves][256], smax[kRangeWaves][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double mn[4], mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mn[j] = __builtin_huge_val();
    mx[j] = -__builtin_huge_val();
  }
  for (int t = blockIdx.x * kRangeWaves + wave; t < T; t += gridDim.x * kRangeWaves) {
    int ec[4];
    double cand[4];
    rt::token_logits(P, KB, bias, T, E, t, ec, cand);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cand[j] == cand[j]) {
        mn[j] = cand[j] < mn[j] ? cand[j] : mn[j];
        mx[j] = cand[j] > mx[j] ? cand[j] : mx[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      smin[wave][e] = mn[j];
      smax[wave][e] = mx[j];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64 * kRangeWaves) {
    double a = smin[0][e], b = smax[0][e];
    for (int w = 1; w < kRangeWaves; ++w) {
      a = smin[w][e] < a ? smin[w][e] : a;
      b = smax[w][e] > b ? smax[w][e] : b;
    }
    if (a <= b) {  // the block saw a finite logit of expert e
      atomic_min_f64(lo + e, a);
      atomic_max_f64(hi + e, b);
    }
  }
}

template <int XDT>
hipError_t launch_logits_x(const void* x, const float* Wr, int T, int H, int E,
                           const RoutePlan& p, double* P, hipStream_t s) {
  const int TT = (T + rt::kTT - 1) / rt::kTT;
  dim3 grid(TT * p.eg * p.kb), block(64 * p.ks);
  const size_t smem = p.ks > 1 ? sizeof(double) * p.ks * p.ntw * 4 * 64 : 0;
  switch (p.ntw) {
    case 1:
      hipLaunchKernelGGL((route_logits_kernel<XDT, 1>), grid, block, smem, s, x, Wr, T, H, E, p.eg,
                         p.ks, p.cpw, P);
      break;
    case 2:
      hipLaunchKernelGGL((route_logits_kernel<XDT, 2>), grid, block, smem, s, x, Wr, T, H, E, p.eg,
                         p.ks, p.cpw, P);
      break;
    case 3:
      hipLaunchKernelGGL((route_logits_kernel<XDT, 3>), grid, block, smem, s, x, Wr, T, H, E, p.eg,
                         p.ks, p.cpw, P);
      break;
    default:
      hipLaunchKernelGGL((route_logits_kernel<XDT, 4>), grid, block, smem, s, x, Wr, T, H, E, p.eg,
                         p.ks, p.cpw, P);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_logits(const void* x, int xdt, const float* Wr, int T, int H, int E,
                               double* P, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const RoutePlan p = route_plan(T, H, E);
  return xdt == MOE_BF16 ? launch_logits_x<MOE_BF16>(x, Wr, T, H, E, p, P, s)
                         : launch_logits_x<MOE_F32>(x, Wr, T, H, E, p, P, s);
}

hipError_t launch_route_topk(const double* P, int KB, const float* b, int T, int E, int k,
                             int32_t* ids, float* w, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + kTopkThreads / 64 - 1) / (kTopkThreads / 64));
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(kTopkThreads), 0, s, P, KB, b, T, E, k, ids, w,
                     logits);
  return hipGetLastError();
}

hipError_t launch_route_topk_q(const double* P, int KB, const float* b, int T, int E, int k,
                               const float* qscale, const int32_t* qzero, int32_t* ids, float* w,
                               float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + kTopkThreads / 64 - 1) / (kTopkThreads / 64));
  hipLaunchKernelGGL(route_topk_q_kernel, grid, dim3(kTopkThreads), 0, s, P, KB, b, T, E, k, qscale,
                     qzero, ids, w, logits);
  return hipGetLastError();
}

hipError_t launch_logit_range(const double* P, int KB, const float* b, int T, int E, double* lo,
                              double* hi, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int blocks = (T + 16 * kRangeWaves - 1) / (16 * kRangeWaves);  // ~16 tokens per wavefront
  if (blocks > 512) blocks = 512;
  hipLaunchKernelGGL(logit_range_kernel, dim3(blocks), dim3(64 * kRangeWaves), 0, s, P, KB, b, T, E,
                     lo, hi);
  return hipGetLastError();
}

hipError_t launch_route(const void* x, int xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* logits, double* P,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipError_t e = launch_route_logits(x, xdt, Wr, T, H, E, P, s);
  if (e != hipSuccess) return e;
  return launch_route_topk(P, route_plan(T, H, E).kb, b, T, E, k, ids, w, logits, s);
}

}  // namespace moeq
