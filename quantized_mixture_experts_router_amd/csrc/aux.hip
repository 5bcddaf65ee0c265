// Helper kernels of the layer: expert-input gather (optionally quantised per
// token to int8), per-row int8 quantisation of h, split-K reduction and the
// top-k weighted combine.
//
// Per-token dynamic int8 activations: MoE mixed-precision notes, sections
// 2.1-2.2 (expert inputs quantised per token at run time; absmax scale).
// Weighted combine: Baidu Cloud quantized-MoE article, expert routing
// section (output = sum of the top-k weights times the expert outputs).
#include "common.h"
#include "rows_dev.h"

namespace moeq {

namespace {

using namespace rows;

constexpr int kThreads = 256;

// ===========================================================================
// Per-token int8 quantisation and input gathering
// ===========================================================================
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

// one block per sorted row r: a16[r] = x[perm[r]] (fp16), or its int8 codes;
// each thread moves 8 columns at a time (H % 8 == 0, x 16-byte aligned)
__global__ __launch_bounds__(kThreads) void gather_a_kernel(const void* __restrict__ x, int dt,
                                                          const int32_t* __restrict__ perm, int T,
                                                          int H,
                                                          int quant, f16* __restrict__ a16,
                                                          float* __restrict__ ascale) {
  __shared__ float s_red[kThreads / 64];
  const int r = blockIdx.x;
  const int t = perm[r];
  f16* dst = a16 + (size_t)r * H;
  if ((unsigned)t >= (unsigned)T) {
    // a slot the permutation left unused (dropped assignments): never read x
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) store8_f16(dst + c, z);
    if (quant && threadIdx.x == 0) ascale[r] = 0.f;
    return;
  }
  const size_t base = (size_t)t * H;
  if (quant) {
    float m = 0.f;
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) {
      float v[8];
      load8(x, dt, base + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float s = __fdiv_rn(amax, 127.f);
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) {
      float v[8];
      load8(x, dt, base + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = quant_i8(v[q], s);
      store8_f16(dst + c, v);
    }
    if (threadIdx.x == 0) ascale[r] = s;
  } else {
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) {
      float v[8];
      load8(x, dt, base + c, v);
      store8_f16(dst + c, v);
    }
  }
}

// Block-wide absmax of a row, 8 columns per thread at a time.
__device__ inline float row_absmax8(const void* x, int dt, size_t base, int cols) {
  __shared__ float s_red[kThreads / 64];
  float m = 0.f;
  for (int c = 8 * threadIdx.x; c < cols; c += 8 * kThreads) {
    float v[8];
    load8(x, dt, base + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// h (fp32 [R, I], I % 8 == 0) -> int8 codes held as fp16, per-row scales
__global__ __launch_bounds__(kThreads) void quant_rows_f32_kernel(const float* __restrict__ h,
                                                                int I, f16* __restrict__ h16,
                                                                float* __restrict__ hscale) {
  const int r = blockIdx.x;
  const size_t base = (size_t)r * I;
  const float s = __fdiv_rn(row_absmax8(h, MOE_F32, base, I), 127.f);
  for (int c = 8 * threadIdx.x; c < I; c += 8 * kThreads) {
    float v[8];
    load8(h, MOE_F32, base + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = quant_i8(v[q], s);
    store8_f16(h16 + base + c, v);
  }
  if (threadIdx.x == 0) hscale[r] = s;
}

// standalone per-row int8 quantisation; vec (cols % 8 == 0, v 16-byte and q
// 8-byte aligned) moves 8 columns per load, otherwise one element at a time
__global__ __launch_bounds__(kThreads) void act_quant_i8_kernel(const void* __restrict__ v, int dt,
                                                              int cols, int vec,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ sc) {
  const int r = blockIdx.x;
  const size_t base = (size_t)r * cols;
  float amax;
  if (vec) {
    amax = row_absmax8(v, dt, base, cols);
  } else {
    amax = row_absmax(v, dt, base, cols);
  }
  const float s = __fdiv_rn(amax, 127.f);
  if (vec) {
    for (int c = 8 * threadIdx.x; c < cols; c += 8 * kThreads) {
      float f[8];
      load8(v, dt, base + c, f);
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        w[j >> 2] |= ((uint32_t)(uint8_t)(int8_t)quant_i8(f[j], s)) << (8 * (j & 3));
      *reinterpret_cast<u32x2*>(q + base + c) = u32x2{w[0], w[1]};
    }
  } else {
    for (int c = threadIdx.x; c < cols; c += kThreads)
      q[base + c] = (int8_t)quant_i8(load_val(v, dt, base + c), s);
  }
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


}  // namespace

hipError_t launch_gather_a(const void* x, int xdt, const int32_t* perm, int T, int k, int H,
                           int quant, f16* a16, float* ascale, hipStream_t s) {
  const int R = T * k;
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_a_kernel, dim3(R), dim3(kThreads), 0, s, x, xdt, perm, T, H, quant,
                     a16, ascale);
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
  const int vec = cols % 8 == 0 && ((uintptr_t)v % 16) == 0 && ((uintptr_t)q % 8) == 0;
  hipLaunchKernelGGL(act_quant_i8_kernel, dim3(rows), dim3(kThreads), 0, s, v, dt, cols, vec, q, sc);
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


// Streaming read (measurement aid): thread t of block b reads the 16-byte
// chunks b*256 + t + j*256*blocks and folds them into one XOR word per block.
namespace {

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[4];
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  // eight loads in flight per thread
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, int nontemporal, uint32_t* sink,
                              hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(MOE_STREAM_BLOCKS), dim3(256), 0, s,
                       (const u32x4*)src, n16, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(MOE_STREAM_BLOCKS), dim3(256), 0, s,
                       (const u32x4*)src, n16, sink);
  return hipGetLastError();
}

}  // namespace moeq
