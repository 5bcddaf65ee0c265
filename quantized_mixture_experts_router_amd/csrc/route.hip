// Router logits + top-k + softmax over the selected logits.
//
// Method: Baidu Cloud article on quantized MoE LLM inference, "expert
// routing" section (router linear -> top-k -> softmax over the top-k ->
// weighted sum); "Sparse activation ... GPT-4's 2% activation", section 2.2
// (keep the K highest of E logits). The router stays unquantised (mixed-
// precision notes, section 2.1: int8 logits lose the small gaps between
// experts), so logits are accumulated in fp64: products of bf16/fp32 inputs
// with fp32 weights are exact in fp64 and the sum carries ~1e-16 relative
// error, far below the 1e-6 gap at which a token counts as a near-tie.
#include "common.h"

namespace moeq {

namespace {

constexpr int kThreads = 256;
constexpr int kTB = 16;   // tokens per block
constexpr int kHC = 16;   // hidden chunk staged in LDS
constexpr int kMaxE = 512;
constexpr int kInvalid = 0x7fffffff;

__device__ inline double load_x(const void* x, int xdt, size_t idx) {
  if (xdt == MOE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)x)[idx] << 16;
    return (double)__uint_as_float(u);
  }
  return (double)((const float*)x)[idx];
}

struct StageBufs {
  double xs[kTB][kHC + 1];
  float ws[kMaxE][kHC + 1];
};
constexpr size_t kStageBytes = sizeof(StageBufs);
constexpr size_t kLogitBytes = sizeof(double) * kTB * (kMaxE + 1);
constexpr size_t kSmemBytes = kStageBytes > kLogitBytes ? kStageBytes : kLogitBytes;

// One block: kTB tokens x all E experts. Thread (tg = tid / 64, eg = tid % 64)
// owns tokens 4*tg .. 4*tg+3 and experts eg, eg+64, eg+128, ... (< E).
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* __restrict__ x, int xdt, const float* __restrict__ Wr,
    const float* __restrict__ bias, int T, int H, int E, int k, int32_t* __restrict__ ids_out,
    float* __restrict__ w_out, float* __restrict__ logits_out, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];
  StageBufs& st = *reinterpret_cast<StageBufs*>(smem);
  double (*lg)[kMaxE + 1] = reinterpret_cast<double (*)[kMaxE + 1]>(smem);

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTB;
  const int tg = tid / 64, eg = tid % 64;
  const int EPT = (E + 63) / 64;  // experts per thread (<= 8)

  double acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;

  for (int h0 = 0; h0 < H; h0 += kHC) {
    for (int i = tid; i < kTB * kHC; i += kThreads) {
      int tt = i / kHC, hh = i % kHC;
      int t = t0 + tt, h = h0 + hh;
      st.xs[tt][hh] = (t < T && h < H) ? load_x(x, xdt, (size_t)t * H + h) : 0.0;
    }
    for (int i = tid; i < E * kHC; i += kThreads) {
      int e = i / kHC, hh = i % kHC;
      int h = h0 + hh;
      st.ws[e][hh] = h < H ? Wr[(size_t)e * H + h] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int hh = 0; hh < kHC; ++hh) {
      double xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = st.xs[4 * tg + i][hh];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < EPT) {
          int e = eg + 64 * j;
          double wv = e < E ? (double)st.ws[e][hh] : 0.0;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i][j] = fma(xv[i], wv, acc[i][j]);
        }
      }
    }
    __syncthreads();
  }

  // add the bias; logits to LDS (fp64) and optionally to global (fp32)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < EPT) {
      int e = eg + 64 * j;
      if (e < E) {
        double bv = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int tt = 4 * tg + i;
          double v = acc[i][j] + bv;
          lg[tt][e] = v;
          int t = t0 + tt;
          if (logits_out && t < T) logits_out[(size_t)t * E + e] = (float)v;
        }
      }
    }
  }
  __syncthreads();

  // top-k: wave w handles tokens 4w .. 4w+3
  const int wave = tid / 64, lane = tid % 64;
  for (int q = 0; q < 4; ++q) {
    const int tt = wave * 4 + q;
    const int t = t0 + tt;
    if (t >= T) break;
    uint32_t taken = 0;
    bool nan_seen = false;
    double my_v = 0.0, top_v = 0.0;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      double bv = 0.0;
      int bi = kInvalid;
      for (int j = 0; j < EPT; ++j) {
        int e = lane + 64 * j;
        if (e < E && !((taken >> j) & 1u)) {
          double v = lg[tt][e];
          if (v != v) nan_seen = true;
          if (bi == kInvalid || v > bv) {  // increasing e: ties keep the lower index
            bv = v;
            bi = e;
          }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        double ov = __shfl_xor(bv, off);
        int oi = __shfl_xor(bi, off);
        bool better = oi != kInvalid &&
                      (bi == kInvalid || ov > bv || (ov == bv && oi < bi));
        if (better) {
          bv = ov;
          bi = oi;
        }
      }
      if (r == 0) top_v = bv;
      if (lane == r) {
        my_v = bv;
        my_i = bi;
      }
      if (bi != kInvalid && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    if (nan_seen && flags) atomicOr(flags, (uint32_t)MOE_FLAG_NAN_LOGIT);
    double ex = lane < k ? exp(my_v - top_v) : 0.0;
    double den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (lane < k) {
      ids_out[(size_t)t * k + lane] = my_i;
      w_out[(size_t)t * k + lane] = (float)(ex / den);
    }
  }
}

}  // namespace

hipError_t launch_route(const void* x, int xdt, const float* Wr, const float* b, int T, int H,
                        int E, int k, int32_t* ids, float* w, float* logits, uint32_t* flags,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + kTB - 1) / kTB);
  hipLaunchKernelGGL(route_kernel, grid, dim3(kThreads), 0, s, x, xdt, Wr, b, T, H, E, k, ids, w,
                     logits, flags);
  return hipGetLastError();
}

}  // namespace moeq
