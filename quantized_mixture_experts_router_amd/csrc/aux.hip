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

// Block-wide maximum of a per-thread value (256 threads).
__device__ inline float block_max(float m) {
  __shared__ float s_red[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
}

// one block per sorted row r: a16[r] = x[perm[r]] (fp16), or its int8 codes
// held as fp16 (a16) and/or as bytes with their 64-column sums (a8, asum:
// the int8 GEMM's operands; R rows); each thread moves 8 columns at a time
// (H % 8 == 0, x 16-byte aligned). With int8 codes and NC > 0 a thread keeps
// its NC chunks of 8 columns in registers between the absmax and the
// quantisation (H <= 2048 NC), so the row is read once.
template <int NC>
__global__ __launch_bounds__(kThreads) void gather_a_kernel(const void* __restrict__ x, int dt,
                                                          const int32_t* __restrict__ perm, int T,
                                                          int H,
                                                          int quant, f16* __restrict__ a16,
                                                          float* __restrict__ ascale,
                                                          int8_t* __restrict__ a8,
                                                          float* __restrict__ asum, int R,
                                                          uint32_t* __restrict__ flags) {
  __shared__ float s_red[kThreads / 64];
  const int r = blockIdx.x;
  const int t = perm[r];
  f16* dst = a16 ? a16 + (size_t)r * H : nullptr;
  if ((unsigned)t >= (unsigned)T) {
    // a slot the permutation left unused (dropped assignments): never read x
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) {
      if (dst) store8_f16(dst + c, z);
      if (a8) store_sum64(asum, R, r, c, store8_i8p(a8 + (size_t)r * H + c, z));
    }
    if (quant && threadIdx.x == 0) ascale[r] = 0.f;
    return;
  }
  const size_t base = (size_t)t * H;
  if (quant && NC > 0) {
    float v[NC > 0 ? NC : 1][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = 8 * (threadIdx.x + kThreads * j);
      if (c < H) {
        load8(x, dt, base + c, v[j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[j][q]));
      }
    }
    const float s = __fdiv_rn(block_max(m), 127.f);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = 8 * (threadIdx.x + kThreads * j);
      if (c < H) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[j][q] = quant_i8(v[j][q], s);
        if (dst) store8_f16(dst + c, v[j]);
        if (a8) store_sum64(asum, R, r, c, store8_i8p(a8 + (size_t)r * H + c, v[j]));
      }
    }
    if (threadIdx.x == 0) ascale[r] = s;
  } else if (quant) {
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
      if (dst) store8_f16(dst + c, v);
      if (a8) store_sum64(asum, R, r, c, store8_i8p(a8 + (size_t)r * H + c, v));
    }
    if (threadIdx.x == 0) ascale[r] = s;
  } else {
    bool over = false;
    for (int c = 8 * threadIdx.x; c < H; c += 8 * kThreads) {
      float v[8];
      load8(x, dt, base + c, v);
      over |= store8_f16(dst + c, v);
    }
    if (over && flags) atomicOr(flags, (uint32_t)MOE_FLAG_FP16_RANGE);
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

// h (fp32 [R, I], I % 8 == 0) -> int8 codes held as fp16 (h16) and/or as
// bytes with their 64-column sums (h8, hsum), per-row scales. NC > 0: each
// thread keeps its NC chunks of 8 columns in registers between the absmax
// and the quantisation (I <= 2048 NC), so the row is read once; NC == 0:
// two passes over memory.
template <int NC>
__global__ __launch_bounds__(kThreads) void quant_rows_f32_kernel(const float* __restrict__ h,
                                                                int I, f16* __restrict__ h16,
                                                                float* __restrict__ hscale,
                                                                int8_t* __restrict__ h8,
                                                                float* __restrict__ hsum, int R) {
  const int r = blockIdx.x;
  const size_t base = (size_t)r * I;
  if constexpr (NC > 0) {
    float v[NC][8];
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = 8 * (threadIdx.x + kThreads * j);
      if (c < I) {
        load8(h, MOE_F32, base + c, v[j]);
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[j][q]));
      }
    }
    const float s = __fdiv_rn(block_max(m), 127.f);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = 8 * (threadIdx.x + kThreads * j);
      if (c < I) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[j][q] = quant_i8(v[j][q], s);
        if (h16) store8_f16(h16 + base + c, v[j]);
        if (h8) store_sum64(hsum, R, r, c, store8_i8p(h8 + base + c, v[j]));
      }
    }
    if (threadIdx.x == 0) hscale[r] = s;
  } else {
    const float s = __fdiv_rn(row_absmax8(h, MOE_F32, base, I), 127.f);
    for (int c = 8 * threadIdx.x; c < I; c += 8 * kThreads) {
      float v[8];
      load8(h, MOE_F32, base + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = quant_i8(v[q], s);
      if (h16) store8_f16(h16 + base + c, v);
      if (h8) store_sum64(hsum, R, r, c, store8_i8p(h8 + base + c, v));
    }
    if (threadIdx.x == 0) hscale[r] = s;
  }
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
  const int R = (int)(split_stride / H);  // T * k rows of Y
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    // a dropped assignment (out-of-range expert id), or a caller's inv entry
    // outside Y's rows: no row of Y is read for it
    if (r < 0 || r >= R) continue;
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

// out[t] = sum_j w[t,j] * sum_s yp[s][inv[t*k+j]] over ns partial planes:
// block (token t, 16 columns), wavefront q the 4 columns 4q..4q+3 of them,
// lane l the planes l, l + 64, ...; then a butterfly over the 64 lanes.
// The order of every sum is fixed, so results are the same run to run.
__global__ __launch_bounds__(kThreads) void combine_slices_kernel(const float* __restrict__ yp,
                                                                int ns, size_t plane,
                                                                const float* __restrict__ w,
                                                                const int32_t* __restrict__ inv,
                                                                int H, int k, void* __restrict__ out,
                                                                int out_dt) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 16 + 4 * q;
  const int R = (int)(plane / H);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    if (r < 0 || r >= R) continue;
    const float wt = w[(size_t)t * k + j];
    const float* src = yp + (size_t)r * H + c;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    for (int s = lane; s < ns; s += 64) y += *reinterpret_cast<const f32x4*>(src + s * plane);
    acc += wt * y;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  if (lane != 0) return;
  if (out_dt == MOE_F32) {
    *reinterpret_cast<f32x4*>((float*)out + (size_t)t * H + c) = acc;
  } else {
    uint16_t* o = (uint16_t*)out + (size_t)t * H + c;
    o[0] = f32_to_bf16_rne(acc[0]);
    o[1] = f32_to_bf16_rne(acc[1]);
    o[2] = f32_to_bf16_rne(acc[2]);
    o[3] = f32_to_bf16_rne(acc[3]);
  }
}


// ===========================================================================
// Transposed expert inputs for the prefill outlier corrections
// ===========================================================================
// Block (bx, by) copies padded columns [64 bx, +64) x input columns
// [64 by, +64) through a 64 x 64 LDS tile: 16-byte loads along the input
// rows, 16-byte stores along the output rows. Every block scans the E padded
// segment sizes itself (E <= 256, one per thread); block (0, 0) stores them.
// Within a 32-column group, slot 16 h + 4 g + i holds padded row 8 g + 4 h + i,
// the order in which lane half h of a 32 x 32 MFMA holds its rows.
__global__ __launch_bounds__(kThreads) void transpose_pad_kernel(
    const f16* __restrict__ a, int R, int K, const int32_t* __restrict__ offsets, int E,
    f16* __restrict__ at, int rp, int32_t* __restrict__ poff) {
  static_assert(kMaxE <= kThreads, "one expert per thread");
  __shared__ int s_po[kMaxE + 1], s_lo[kMaxE], s_cnt[kMaxE];
  __shared__ int s_ws[kThreads / 64];
  __shared__ __attribute__((aligned(16))) f16 tile[64][72];  // [column][slot]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c32 = 0;
  if (tid < E) {
    const int o0 = offsets[tid], o1 = offsets[tid + 1];
    const int lo = min(max(o0, 0), R);
    const int hi = min(max(o1, lo), R);
    s_lo[tid] = lo;
    s_cnt[tid] = hi - lo;
    c32 = (hi - lo + 31) & ~31;
  }
  int incl = c32;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_ws[wave] = incl;
  __syncthreads();
  int ex = incl - c32;
  for (int w = 0; w < wave; ++w) ex += s_ws[w];
  if (tid < E) s_po[tid] = ex;
  if (tid == E - 1) s_po[E] = ex + c32;
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i <= E; i += kThreads) poff[i] = s_po[i];
  const int total = s_po[E];
  const int p0 = 64 * blockIdx.x, k0 = 64 * blockIdx.y;
  if (p0 >= total) return;  // block-uniform
  for (int q = tid; q < 512; q += kThreads) {
    const int j = q >> 3, c8 = q & 7;  // padded row p0 + j, input columns k0 + 8 c8
    const int p = p0 + j;
    if (p < total) {
      int lo = 0, hi = E;  // s_po[lo] <= p < s_po[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_po[mid] <= p) lo = mid;
        else hi = mid;
      }
      const int row = s_lo[lo] + min(p - s_po[lo], s_cnt[lo] - 1);
      const u32x4 v = *reinterpret_cast<const u32x4*>(a + (size_t)row * K + k0 + 8 * c8);
      const int rho = j & 31;
      const int slot = (j & 32) | (16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        tile[8 * c8 + 2 * t][slot] = __builtin_bit_cast(f16, (uint16_t)(v[t] & 0xffffu));
        tile[8 * c8 + 2 * t + 1][slot] = __builtin_bit_cast(f16, (uint16_t)(v[t] >> 16));
      }
    }
  }
  __syncthreads();
  for (int q = tid; q < 512; q += kThreads) {
    const int kk = q >> 3, c = q & 7;  // input column k0 + kk, slots [8 c, +8)
    if (p0 + 8 * c < total)
      *reinterpret_cast<u32x4*>(at + (size_t)(k0 + kk) * rp + p0 + 8 * c) =
          *reinterpret_cast<const u32x4*>(&tile[kk][8 * c]);
  }
}

}  // namespace

hipError_t launch_transpose_pad(const f16* a, int R, int K, const int32_t* offsets, int E,
                                f16* at, int rp, int32_t* poff, hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3(rp / 64, K / 64), dim3(kThreads), 0, s, a, R, K,
                     offsets, E, at, rp, poff);
  return hipGetLastError();
}

hipError_t launch_combine_slices(const float* yp, int ns, const float* w, const int32_t* inv,
                                 int T, int H, int k, void* out, int out_dt, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const size_t plane = (size_t)T * k * H;
  dim3 grid(H / 16, T);
  hipLaunchKernelGGL(combine_slices_kernel, grid, dim3(kThreads), 0, s, yp, ns, plane, w, inv, H,
                     k, out, out_dt);
  return hipGetLastError();
}

hipError_t launch_gather_a(const void* x, int xdt, const int32_t* perm, int T, int k, int H,
                           int quant, f16* a16, float* ascale, int8_t* a8, float* asum,
                           uint32_t* flags, hipStream_t s) {
  const int R = T * k;
  if (R == 0) return hipSuccess;
  // int8 codes of rows up to 4096 / 16384 columns: the row is read once
  auto kern = !quant || H > 8 * kThreads * 8 ? gather_a_kernel<0>
              : H <= 8 * kThreads * 2        ? gather_a_kernel<2>
                                             : gather_a_kernel<8>;
  hipLaunchKernelGGL(kern, dim3(R), dim3(kThreads), 0, s, x, xdt, perm, T, H, quant, a16, ascale,
                     quant ? a8 : nullptr, asum, R, flags);
  return hipGetLastError();
}

hipError_t launch_quant_rows_f32(const float* h, int R, int I, f16* h16, float* hscale,
                                 int8_t* h8, float* hsum, hipStream_t s) {
  if (R == 0) return hipSuccess;
  // rows of up to 4096 / 16384 columns are read once (kept in registers)
  if (I <= 8 * kThreads * 2)
    hipLaunchKernelGGL(quant_rows_f32_kernel<2>, dim3(R), dim3(kThreads), 0, s, h, I, h16, hscale,
                       h8, hsum, R);
  else if (I <= 8 * kThreads * 8)
    hipLaunchKernelGGL(quant_rows_f32_kernel<8>, dim3(R), dim3(kThreads), 0, s, h, I, h16, hscale,
                       h8, hsum, R);
  else
    hipLaunchKernelGGL(quant_rows_f32_kernel<0>, dim3(R), dim3(kThreads), 0, s, h, I, h16, hscale,
                       h8, hsum, R);
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

// Shaped streaming read (measurement aid): the same XOR fold, with the
// launch shape as a parameter, so the read rate can be measured over block
// counts, block sizes, loads in flight per thread and two layouts:
//  * interleaved (layout 0): thread t of block b reads chunks
//    b*nthr + t + j*nthr*blocks, so the grid sweeps the buffer as one front;
//  * contiguous (layout 1): block b owns one contiguous run of
//    ceil(n16 / blocks) chunks and sweeps it nthr chunks at a time, the way a
//    GEMV block streams its own weight rows.
template <bool NT, int U>
__global__ __launch_bounds__(1024) void stream_read_shaped_kernel(const u32x4* __restrict__ src,
                                                                  size_t n16, int layout,
                                                                  uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[16];
  const size_t nthr = blockDim.x;
  size_t i, stride, end;
  if (layout == 0) {
    i = (size_t)blockIdx.x * nthr + threadIdx.x;
    stride = (size_t)gridDim.x * nthr;
    end = n16;
  } else {
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = min((size_t)blockIdx.x * chunk, n16);
    i = b0 + threadIdx.x;
    stride = nthr;
    end = min(b0 + chunk, n16);
  }
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < end; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  const int nw = blockDim.x / 64;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < nw; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

template <bool NT>
hipError_t launch_shaped(const u32x4* src, size_t n16, int blocks, int waves, int inflight,
                         int layout, uint32_t* sink, hipStream_t s) {
  const dim3 grid(blocks), block(64 * waves);
  switch (inflight) {
    case 1: hipLaunchKernelGGL((stream_read_shaped_kernel<NT, 1>), grid, block, 0, s, src, n16, layout, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_shaped_kernel<NT, 2>), grid, block, 0, s, src, n16, layout, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_shaped_kernel<NT, 4>), grid, block, 0, s, src, n16, layout, sink); break;
    case 8: hipLaunchKernelGGL((stream_read_shaped_kernel<NT, 8>), grid, block, 0, s, src, n16, layout, sink); break;
    default: hipLaunchKernelGGL((stream_read_shaped_kernel<NT, 16>), grid, block, 0, s, src, n16, layout, sink); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read_shaped(const void* src, size_t bytes, int nontemporal, int blocks,
                                     int waves, int inflight, int layout, uint32_t* sink,
                                     hipStream_t s) {
  const size_t n16 = bytes / 16;
  return nontemporal ? launch_shaped<true>((const u32x4*)src, n16, blocks, waves, inflight, layout, sink, s)
                     : launch_shaped<false>((const u32x4*)src, n16, blocks, waves, inflight, layout, sink, s);
}

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
