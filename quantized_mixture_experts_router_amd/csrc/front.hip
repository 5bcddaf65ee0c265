// Fused front of the layer for small batches, run after the logits
// kernel: top-k + softmax of every token, the stable permutation by expert
// and the expert-input gather (optionally quantised per token to int8) in
// one block of 8 wavefronts.
//
// At decode sizes each of these steps is a few microseconds of work but a
// separate launch costs about as much again; one block that runs them back
// to back replaces three launches (top-k, permutation, gather). Used while
// the gathered rows and the logits stay small enough for one CU; larger
// batches take the separate kernels.
#include "permute_dev.h"
#include "route_dev.h"
#include "rows_dev.h"

namespace moeq {

namespace {

constexpr int kFW = 8;         // wavefronts
constexpr int kFT = kFW * 64;  // threads

template <int XDT>
__global__ __launch_bounds__(kFT) void front_kernel(
    const double* __restrict__ P, int KB, const void* __restrict__ x,
    const float* __restrict__ bias, int T, int H, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, uint32_t* __restrict__ flags, int quant,
    f16* __restrict__ a16, float* __restrict__ ascale) {
  // LDS: the permutation's scratch, then copies of the ids, of perm and of
  // the row count, so each phase reads the previous one's results from LDS
  // rather than through memory
  extern __shared__ int32_t smem[];
  const int R = T * k;
  int32_t* s_ids = smem + pm::permute_smem_words(kFW, E);
  int32_t* s_perm = s_ids + R;
  int32_t* s_rows = s_perm + R;
  // 1. top-k + softmax, one wavefront per token
  for (int t = threadIdx.x / 64; t < T; t += kFW)
    rt::topk_token(P, KB, bias, T, E, k, t, ids, w, nullptr, s_ids);
  __syncthreads();
  // 2. permutation
  const uint32_t bits =
      pm::permute_block<kFW>(s_ids, R, k, E, counts, offsets, perm, inv, smem, s_perm, s_rows);
  __syncthreads();
  // 3. gather of the rows the permutation produced
  const int rows_used = *s_rows;
  bool over = false;  // an fp16 expert input out of range
  if (!quant) {
    // every thread moves 8-column chunks of any row; a batch of kU chunks per
    // thread is loaded before any is stored, so one memory round trip covers
    // kU * kFT chunks
    constexpr int kU = 16;
    const int CH = H / 8;
    const int total = rows_used * CH;
    for (int b0 = threadIdx.x; b0 < total; b0 += kFT * kU) {
      u32x4 raw[kU][XDT == MOE_BF16 ? 1 : 2];
      int dsto[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int idx = min(b0 + u * kFT, total - 1);
        const int r = idx / CH, c = idx % CH;
        const size_t src = (size_t)s_perm[r] * H + 8 * c;
        dsto[u] = r * H + 8 * c;
        if (XDT == MOE_BF16) {
          raw[u][0] = *reinterpret_cast<const u32x4*>((const uint16_t*)x + src);
        } else {
          raw[u][0] = *reinterpret_cast<const u32x4*>((const float*)x + src);
          raw[u][XDT == MOE_BF16 ? 0 : 1] = *reinterpret_cast<const u32x4*>((const float*)x + src + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (b0 + u * kFT >= total) break;
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (XDT == MOE_BF16) {
            v[2 * q] = __uint_as_float(raw[u][0][q] << 16);
            v[2 * q + 1] = __uint_as_float(raw[u][0][q] & 0xffff0000u);
          } else {
            v[q] = __uint_as_float(raw[u][0][q]);
            v[4 + q] = __uint_as_float(raw[u][XDT == MOE_BF16 ? 0 : 1][q]);
          }
        }
        over |= rows::store8_f16(a16 + dsto[u], v);
      }
    }
  } else {
    // int8: wavefront w quantises rows w, w + 8, ...
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    for (int r = wave; r < rows_used; r += kFT / 64) {
      const size_t src = (size_t)s_perm[r] * H;
      f16* dst = a16 + (size_t)r * H;
      float m = 0.f;
      for (int c = 8 * lane; c < H; c += 512) {
        float v[8];
        rows::load8(x, XDT, src + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float s = __fdiv_rn(m, 127.f);
      if (lane == 0) ascale[r] = s;
      for (int c = 8 * lane; c < H; c += 512) {
        float v[8];
        rows::load8(x, XDT, src + c, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = rows::quant_i8(v[q], s);
        rows::store8_f16(dst + c, v);
      }
    }
  }
  // the call's flag word starts here
  const bool any_over = __syncthreads_or(over);
  if (threadIdx.x == 0) *flags = bits | (any_over ? (uint32_t)MOE_FLAG_FP16_RANGE : 0u);
}

}  // namespace

// One CU gathers the rows and sums the partial logits: kept to a few
// hundred KB of each.
bool front_fits(int T, int H, int E, int k) {
  return (long)T * k * H * 2 <= (256L << 10) && (long)T * E * route_plan(T, H, E).kb <= 32768;
}

hipError_t launch_front(const double* P, int KB, const void* x, int xdt, const float* b, int T,
                        int H, int E, int k, int32_t* ids, float* w, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv, uint32_t* flags, int quant,
                        f16* a16, float* ascale, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const size_t smem = sizeof(int32_t) * (pm::permute_smem_words(kFW, E) + 2 * (size_t)T * k + 1);
  if (xdt == MOE_BF16)
    hipLaunchKernelGGL(front_kernel<MOE_BF16>, dim3(1), dim3(kFT), smem, s, P, KB, x, b, T, H, E,
                       k, ids, w, counts, offsets, perm, inv, flags, quant, a16, ascale);
  else
    hipLaunchKernelGGL(front_kernel<MOE_F32>, dim3(1), dim3(kFT), smem, s, P, KB, x, b, T, H, E,
                       k, ids, w, counts, offsets, perm, inv, flags, quant, a16, ascale);
  return hipGetLastError();
}

}  // namespace moeq
