// Helper kernels of the layer: expert-input gather (optionally quantised per
// token to int8), per-row int8 quantisation of h, split-K reduction and the
// top-k weighted combine.
//
// Per-token dynamic int8 activations: MoE mixed-precision notes, sections
// 2.1-2.2 (expert inputs quantised per token at run time; absmax scale).
// Weighted combine: Baidu Cloud quantized-MoE article, expert routing
// section (output = sum of the top-k weights times the expert outputs).
#include "common.h"

namespace moeq {

namespace {

constexpr int kThreads = 256;

// ===========================================================================
// Per-token int8 quantisation and input gathering
// ===========================================================================
__device__ inline float load_val(const void* x, int dt, size_t idx) {
  if (dt == MOE_BF16) return __uint_as_float((uint32_t)((const uint16_t*)x)[idx] << 16);
  return ((const float*)x)[idx];
}

// Block-wide absmax of a row (256 threads).
__device__ inline float row_absmax(const void* x, int dt, size_t base, int cols) {
  __shared__ float s_red[kThreads / 64];
  float m = 0.f;
  for (int c = threadIdx.x; c < cols; c += kThreads) m = fmaxf(m, fabsf(load_val(x, dt, base + c)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  return r;
}

// q = clamp(rint(v / s), -127, 127) with IEEE fp32 division; s = absmax / 127.
__device__ inline float quant_i8(float v, float s) {
  if (s == 0.f) return 0.f;
  float q = __builtin_rintf(__fdiv_rn(v, s));
  return fminf(fmaxf(q, -127.f), 127.f);
}

// one block per sorted row r: a16[r] = x[perm[r]] (fp16), or its int8 codes
__global__ __launch_bounds__(kThreads) void gather_a_kernel(const void* __restrict__ x, int dt,
                                                          const int32_t* __restrict__ perm, int H,
                                                          int quant, f16* __restrict__ a16,
                                                          float* __restrict__ ascale) {
  const int r = blockIdx.x;
  const int t = perm[r];
  const size_t base = (size_t)t * H;
  f16* dst = a16 + (size_t)r * H;
  if (quant) {
    float amax = row_absmax(x, dt, base, H);
    float s = __fdiv_rn(amax, 127.f);
    for (int c = threadIdx.x; c < H; c += kThreads) dst[c] = (f16)quant_i8(load_val(x, dt, base + c), s);
    if (threadIdx.x == 0) ascale[r] = s;
  } else {
    for (int c = threadIdx.x; c < H; c += kThreads) dst[c] = (f16)load_val(x, dt, base + c);
  }
}

__global__ __launch_bounds__(kThreads) void quant_rows_f32_kernel(const float* __restrict__ h,
                                                                int I, f16* __restrict__ h16,
                                                                float* __restrict__ hscale) {
  const int r = blockIdx.x;
  const size_t base = (size_t)r * I;
  float amax = row_absmax(h, MOE_F32, base, I);
  float s = __fdiv_rn(amax, 127.f);
  for (int c = threadIdx.x; c < I; c += kThreads) h16[base + c] = (f16)quant_i8(h[base + c], s);
  if (threadIdx.x == 0) hscale[r] = s;
}

__global__ __launch_bounds__(kThreads) void act_quant_i8_kernel(const void* __restrict__ v, int dt,
                                                              int cols, int8_t* __restrict__ q,
                                                              float* __restrict__ sc) {
  const int r = blockIdx.x;
  const size_t base = (size_t)r * cols;
  float amax = row_absmax(v, dt, base, cols);
  float s = __fdiv_rn(amax, 127.f);
  for (int c = threadIdx.x; c < cols; c += kThreads) q[base + c] = (int8_t)quant_i8(load_val(v, dt, base + c), s);
  if (threadIdx.x == 0) sc[r] = s;
}

// ===========================================================================
// Split reduction and weighted combine
// ===========================================================================
__global__ void reduce_splits_kernel(const float* __restrict__ yp, int splits, size_t n,
                                     float* __restrict__ Y) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int q = 0; q < splits; ++q) s += yp[q * n + i];
  Y[i] = s;
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// out[t] = sum_j w[t,j] * sum_s yp[s][inv[t*k+j]]: one thread per (token,
// 4 columns); the partial-sum loads of all slots and splits are independent
// and issued together. Summation order is fixed (deterministic).
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ yp, int splits,
                                                         size_t split_stride,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ inv, int H,
                                                         int k, void* __restrict__ out, int out_dt) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * kThreads + threadIdx.x;
  if (c4 >= H / 4) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    if (r < 0) continue;  // dropped assignment (out-of-range expert id)
    const float wt = w[(size_t)t * k + j];
    const float* src = yp + (size_t)r * H + 4 * c4;
    f32x4 y = *reinterpret_cast<const f32x4*>(src);
#pragma unroll 8
    for (int q = 1; q < splits; ++q) y += *reinterpret_cast<const f32x4*>(src + q * split_stride);
    acc += wt * y;
  }
  if (out_dt == MOE_F32) {
    *reinterpret_cast<f32x4*>((float*)out + (size_t)t * H + 4 * c4) = acc;
  } else {
    uint16_t* o = (uint16_t*)out + (size_t)t * H + 4 * c4;
    o[0] = f32_to_bf16_rne(acc[0]);
    o[1] = f32_to_bf16_rne(acc[1]);
    o[2] = f32_to_bf16_rne(acc[2]);
    o[3] = f32_to_bf16_rne(acc[3]);
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_gather_a(const void* x, int xdt, const int32_t* perm, int R, int H, int quant,
                           f16* a16, float* ascale, hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_a_kernel, dim3(R), dim3(kThreads), 0, s, x, xdt, perm, H, quant, a16,
                     ascale);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f32(const float* h, int R, int I, f16* h16, float* hscale,
                                 hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_f32_kernel, dim3(R), dim3(kThreads), 0, s, h, I, h16, hscale);
  return hipGetLastError();
}

hipError_t launch_act_quant_i8(const void* v, int dt, int rows, int cols, int8_t* q, float* sc,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(act_quant_i8_kernel, dim3(rows), dim3(kThreads), 0, s, v, dt, cols, q, sc);
  return hipGetLastError();
}

hipError_t launch_reduce_splits(const float* yp, int splits, size_t n, float* Y, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, yp,
                     splits, n, Y);
  return hipGetLastError();
}

hipError_t launch_combine(const float* yp, int splits, const float* w, const int32_t* inv, int T,
                          int H, int k, void* out, int out_dt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  size_t stride = (size_t)T * k * H;
  dim3 grid((H / 4 + kThreads - 1) / kThreads, T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, yp, splits, stride, w, inv, H, k,
                     out, out_dt);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moeq
