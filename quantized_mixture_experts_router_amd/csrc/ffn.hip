// Grouped expert FFN: gather/quantise expert inputs, gate/up + SwiGLU,
// (quantise h), down projection, split reduction and the weighted combine.
//
// Expert FFN: three matrices per expert, gate/up/down ("AlphaQ" blog,
// section 2.2; MoE mixed-precision notes, section 3.3), in the gated SwiGLU
// form h = silu(a Wg^T) * (a Wu^T), y = h Wd^T. SwiGLU is fused into the
// gate/up epilogue (the notes fuse the expert activation into the linear,
// section 3.6). Only the experts a token was routed to are read ("Sparse
// activation ... 2% activation", section 3.1: the saving is in bandwidth).
// Optional per-token int8 expert inputs (mixed-precision notes, 2.1-2.2).
//
// Two kernel families share the tile layout and the in-register decoding:
//  * decode (few rows per expert): a block is 4 wavefronts on the same 32-row
//    token tile and the same 64 weight rows, splitting K; weights stream from
//    HBM straight into registers (16-byte loads per lane, coalesced 1 KiB per
//    wave), are decoded to fp16 and fed to v_mfma_f32_32x32x16_f16 with the
//    token rows padded to 32. The 4 partial sums meet in LDS.
//  * prefill (many rows per expert): a block owns 128 token rows x 4 weight
//    tiles pairs; the token tile is staged in LDS (double-buffered) and shared
//    by the 4 wavefronts; each wavefront streams its own weight rows into
//    registers.
// Tasks are (expert, n-tile, m-tile), expert-major, so blocks that share
// weight tiles run together; the task list is derived inside each block from
// the segment offsets, so no host synchronisation is needed.
#include "common.h"
#include "deq.h"

namespace moeq {

namespace {

constexpr int kThreads = 256;

__device__ inline f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Row of accumulator register r for lane `lane` in a 32x32 MFMA output tile.
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct FfnArgs {
  const moe_packed_expert* experts;
  const int32_t* offsets;
  int E;
  int K;          // reduction dim (H for gate/up, I for down)
  int N;          // outputs per expert (I for gate/up, H for down)
  int gu;         // 1: gate/up + SwiGLU; 0: down
  const f16* a;   // [R, K] rows in sorted order
  const float* ascale;  // per-row scale (int8 inputs) or null
  void* out;      // gate/up: h [R, N] (f16 or f32); down: [splits][R][N] f32
  int out_f32;
  int R;
  int splits;
};

// ---------------------------------------------------------------------------
// Task lookup: tasks of expert e = ceil(count_e / BM) * NB, expert-major, then
// n-tile, then m-tile. Every thread of the block gets the result.
// ---------------------------------------------------------------------------
struct Task {
  int e, row0, mcount, nt;
};

__device__ bool find_task(const int32_t* __restrict__ offsets, int E, int BM, int NB, int L,
                          Task& task) {
  __shared__ int s_wsum[kThreads / 64];
  __shared__ int s_res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_res[0] = -1;
  // each thread: experts 2*tid, 2*tid+1
  int cnt[2], nt_[2];
  int local = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    int e = 2 * tid + q;
    int c = e < E ? offsets[e + 1] - offsets[e] : 0;
    cnt[q] = c;
    nt_[q] = ((c + BM - 1) / BM) * NB;
    local += nt_[q];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += s_wsum[w];
  int start = wbase + incl - local;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (L >= start && L < start + nt_[q]) {
      int e = 2 * tid + q;
      int rel = L - start;
      int mt = (cnt[q] + BM - 1) / BM;
      int nt = rel / mt, mi = rel % mt;
      s_res[0] = e;
      s_res[1] = offsets[e] + mi * BM;
      s_res[2] = min(BM, cnt[q] - mi * BM);
      s_res[3] = nt;
    }
    start += nt_[q];
  }
  __syncthreads();
  task.e = s_res[0];
  task.row0 = s_res[1];
  task.mcount = s_res[2];
  task.nt = s_res[3];
  return task.e >= 0;
}

// Epilogue for one accumulator pair element.
__device__ inline void store_gu(const FfnArgs& a, int row, int col, float g, float u) {
  float sc = a.ascale ? a.ascale[row] : 1.0f;
  float h = silu_mul(g * sc, u * sc);
  if (a.out_f32)
    reinterpret_cast<float*>(a.out)[(size_t)row * a.N + col] = h;
  else
    reinterpret_cast<f16*>(a.out)[(size_t)row * a.N + col] = (f16)h;
}

__device__ inline void store_dn(const FfnArgs& a, int split, int row, int col, float y) {
  float sc = a.ascale ? a.ascale[row] : 1.0f;
  reinterpret_cast<float*>(a.out)[((size_t)split * a.R + row) * a.N + col] = y * sc;
}

// ===========================================================================
// Decode family
// ===========================================================================
template <class F>
__device__ void decode_body(const FfnArgs& a, const Task& t, const moe_packed_expert& ex,
                            float* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, kh = lane >> 5;
  const int KTn = a.K / F::KT;
  const int NE = a.K / F::GE;
  const uint8_t* codes = (const uint8_t*)(a.gu ? ex.gu_codes : ex.dn_codes);
  const uint8_t* params = (const uint8_t*)(a.gu ? ex.gu_params : ex.dn_params);
  const int rt0 = 2 * t.nt;  // gate tile (gu) or first row tile (down)
  const uint8_t* c0 = codes + (size_t)rt0 * KTn * 1024 + lane * 16;
  const uint8_t* c1 = c0 + (size_t)KTn * 1024;
  const uint8_t* p0 = params + ((size_t)rt0 * NE * 32 + n) * F::EB;
  const uint8_t* p1 = p0 + (size_t)NE * 32 * F::EB;

  const int split = blockIdx.y;
  const int per = (KTn + a.splits - 1) / a.splits;
  const int kb = split * per, ke = min(KTn, kb + per);

  const bool arow = n < t.mcount;
  const f16* ap = a.a + (size_t)(t.row0 + (arow ? n : 0)) * a.K + kh * F::SPAN;

  f32x16 acc0 = {}, acc1 = {};
  for (int kt = kb + wave; kt < ke; kt += 4) {
    u32x4 w0 = *reinterpret_cast<const u32x4*>(c0 + (size_t)kt * 1024);
    u32x4 w1 = *reinterpret_cast<const u32x4*>(c1 + (size_t)kt * 1024);
    const int ei = (kt * F::KT + kh * F::SPAN) / F::GE;
    PBuf<F::EB> q0, q1;
    q0.load(p0 + (size_t)ei * 32 * F::EB);
    q1.load(p1 + (size_t)ei * 32 * F::EB);
    f16x8 av[F::STEPS];
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
      if (arow)
        av[s] = *reinterpret_cast<const f16x8*>(ap + (size_t)kt * F::KT + 8 * s);
      else
        av[s] = f16x8{};
    }
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
      f16x8 b0 = dequant_step<F>(w0, q0, s);
      f16x8 b1 = dequant_step<F>(w1, q1, s);
      acc0 = mfma32(av[s], b0, acc0);
      acc1 = mfma32(av[s], b1, acc1);
    }
  }

  // reduce the 4 wavefronts' partial sums: red[w][m][r][lane]
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    red[((wave * 2 + 0) * 16 + r) * 64 + lane] = acc0[r];
    red[((wave * 2 + 1) * 16 + r) * 64 + lane] = acc1[r];
  }
  __syncthreads();
  // wavefront w finalises registers r = 4w .. 4w+3
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * wave + rr;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      v0 += red[((w * 2 + 0) * 16 + r) * 64 + lane];
      v1 += red[((w * 2 + 1) * 16 + r) * 64 + lane];
    }
    const int i = acc_row(r, lane);
    if (i < t.mcount) {
      const int row = t.row0 + i;
      if (a.gu) {
        store_gu(a, row, 32 * t.nt + n, v0, v1);
      } else {
        store_dn(a, split, row, 64 * t.nt + n, v0);
        store_dn(a, split, row, 64 * t.nt + 32 + n, v1);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void ffn_decode_kernel(FfnArgs a) {
  __shared__ float red[4 * 2 * 16 * 64];
  const int NB = a.gu ? a.N / 32 : a.N / 64;
  Task t;
  if (!find_task(a.offsets, a.E, 32, NB, blockIdx.x, t)) return;
  const moe_packed_expert ex = a.experts[t.e];
  const int fid = a.gu ? fmt_id(ex.gu_fmt, ex.gu_bits, ex.gu_group)
                       : fmt_id(ex.dn_fmt, ex.dn_bits, ex.dn_group);
  switch (fid) {
    case F_A4G16: decode_body<Fmt<MOE_W_ASYM, 4, 16>>(a, t, ex, red); break;
    case F_A4G32: decode_body<Fmt<MOE_W_ASYM, 4, 32>>(a, t, ex, red); break;
    case F_A4G64: decode_body<Fmt<MOE_W_ASYM, 4, 64>>(a, t, ex, red); break;
    case F_A4G128: decode_body<Fmt<MOE_W_ASYM, 4, 128>>(a, t, ex, red); break;
    case F_A2G16: decode_body<Fmt<MOE_W_ASYM, 2, 16>>(a, t, ex, red); break;
    case F_A2G32: decode_body<Fmt<MOE_W_ASYM, 2, 32>>(a, t, ex, red); break;
    case F_A2G64: decode_body<Fmt<MOE_W_ASYM, 2, 64>>(a, t, ex, red); break;
    case F_A2G128: decode_body<Fmt<MOE_W_ASYM, 2, 128>>(a, t, ex, red); break;
    case F_E4G16: decode_body<Fmt<MOE_W_E2M1, 4, 16>>(a, t, ex, red); break;
    case F_E4G32: decode_body<Fmt<MOE_W_E2M1, 4, 32>>(a, t, ex, red); break;
    case F_E4G64: decode_body<Fmt<MOE_W_E2M1, 4, 64>>(a, t, ex, red); break;
    case F_E4G128: decode_body<Fmt<MOE_W_E2M1, 4, 128>>(a, t, ex, red); break;
    default: break;
  }
}

// ===========================================================================
// Prefill family
// ===========================================================================
constexpr int kBM = 128;
constexpr int kMT = kBM / 32;        // 32-row sub-tiles per block tile
constexpr int kMaxKT = 128;          // largest K tile (2-bit formats)
constexpr int kLdsStride = kMaxKT + 8;  // halves per staged row (+16 B pad)

template <class F>
__device__ void prefill_body(const FfnArgs& a, const Task& t, const moe_packed_expert& ex,
                             f16* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, kh = lane >> 5;
  const int KTn = a.K / F::KT;
  const int NE = a.K / F::GE;
  constexpr int STR = F::KT + 8;  // LDS row stride (halves)
  const uint8_t* codes = (const uint8_t*)(a.gu ? ex.gu_codes : ex.dn_codes);
  const uint8_t* params = (const uint8_t*)(a.gu ? ex.gu_params : ex.dn_params);
  // gate/up: wave w owns output tile 4*nt + w = row tiles (2j, 2j+1);
  // down: wave w owns row tiles 8*nt + 2w, +1.
  const int rt0 = a.gu ? 2 * (4 * t.nt + wave) : 8 * t.nt + 2 * wave;
  const bool wave_on = rt0 + 1 < (a.gu ? 2 * (a.N / 32) : a.N / 32) + (a.gu ? 0 : 1) &&
                       (a.gu || rt0 < a.N / 32);
  const uint8_t* c0 = codes + (size_t)rt0 * KTn * 1024 + lane * 16;
  const uint8_t* c1 = c0 + (size_t)KTn * 1024;
  const uint8_t* p0 = params + ((size_t)rt0 * NE * 32 + n) * F::EB;
  const uint8_t* p1 = p0 + (size_t)NE * 32 * F::EB;
  const bool has1 = a.gu || (rt0 + 1) < a.N / 32;

  // A staging: kBM rows x KT halves = kBM * KT/8 chunks of 16 B
  constexpr int CPR = F::KT / 8;               // chunks per row
  constexpr int CPT = kBM * CPR / kThreads;    // chunks per thread
  f16x8 areg[CPT];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int ch = tid + i * kThreads;
      int r = ch / CPR, c = ch % CPR;
      if (r < t.mcount)
        areg[i] = *reinterpret_cast<const f16x8*>(a.a + (size_t)(t.row0 + r) * a.K +
                                                  (size_t)kt * F::KT + 8 * c);
      else
        areg[i] = f16x8{};
    }
  };
  auto store_a = [&](int buf) {
    f16* base = lds + buf * (kBM * kLdsStride);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      int ch = tid + i * kThreads;
      int r = ch / CPR, c = ch % CPR;
      *reinterpret_cast<f16x8*>(base + r * STR + 8 * c) = areg[i];
    }
  };

  f32x16 acc[kMT][2];
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi) {
    acc[mi][0] = f32x16{};
    acc[mi][1] = f32x16{};
  }

  u32x4 w0 = {}, w1 = {};
  PBuf<F::EB> q0, q1;
  auto load_b = [&](int kt) {
    if (wave_on) {
      w0 = *reinterpret_cast<const u32x4*>(c0 + (size_t)kt * 1024);
      const int ei = (kt * F::KT + kh * F::SPAN) / F::GE;
      q0.load(p0 + (size_t)ei * 32 * F::EB);
      if (has1) {
        w1 = *reinterpret_cast<const u32x4*>(c1 + (size_t)kt * 1024);
        q1.load(p1 + (size_t)ei * 32 * F::EB);
      }
    }
  };

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();
  for (int kt = 0; kt < KTn; ++kt) {
    const int buf = kt & 1;
    u32x4 cw0 = w0, cw1 = w1;
    PBuf<F::EB> cq0 = q0, cq1 = q1;
    if (kt + 1 < KTn) {
      load_a(kt + 1);
      load_b(kt + 1);
    }
    if (wave_on) {
      const f16* base = lds + buf * (kBM * kLdsStride);
#pragma unroll
      for (int s = 0; s < F::STEPS; ++s) {
        f16x8 b0 = dequant_step<F>(cw0, cq0, s);
        f16x8 b1 = has1 ? dequant_step<F>(cw1, cq1, s) : f16x8{};
#pragma unroll
        for (int mi = 0; mi < kMT; ++mi) {
          f16x8 av = *reinterpret_cast<const f16x8*>(base + (mi * 32 + n) * STR + kh * F::SPAN + 8 * s);
          acc[mi][0] = mfma32(av, b0, acc[mi][0]);
          acc[mi][1] = mfma32(av, b1, acc[mi][1]);
        }
      }
    }
    if (kt + 1 < KTn) store_a(buf ^ 1);
    __syncthreads();
  }

  if (!wave_on) return;
#pragma unroll
  for (int mi = 0; mi < kMT; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = mi * 32 + acc_row(r, lane);
      if (i < t.mcount) {
        const int row = t.row0 + i;
        if (a.gu) {
          store_gu(a, row, 32 * (4 * t.nt + wave) + n, acc[mi][0][r], acc[mi][1][r]);
        } else {
          store_dn(a, 0, row, 32 * rt0 + n, acc[mi][0][r]);
          if (has1) store_dn(a, 0, row, 32 * (rt0 + 1) + n, acc[mi][1][r]);
        }
      }
    }
  }
}

__device__ inline int xcd_remap(int b, int nblk) {
  const int xcd = b & 7, slot = b >> 3;
  const int q = nblk >> 3, r = nblk & 7;
  return xcd * q + min(xcd, r) + slot;
}

__global__ __launch_bounds__(kThreads) void ffn_prefill_kernel(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) f16 lds[2 * kBM * kLdsStride];
  const int NB = a.gu ? a.N / 128 : (a.N + 255) / 256;
  Task t;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (!find_task(a.offsets, a.E, kBM, NB, L, t)) return;
  const moe_packed_expert ex = a.experts[t.e];
  const int fid = a.gu ? fmt_id(ex.gu_fmt, ex.gu_bits, ex.gu_group)
                       : fmt_id(ex.dn_fmt, ex.dn_bits, ex.dn_group);
  switch (fid) {
    case F_A4G16: prefill_body<Fmt<MOE_W_ASYM, 4, 16>>(a, t, ex, lds); break;
    case F_A4G32: prefill_body<Fmt<MOE_W_ASYM, 4, 32>>(a, t, ex, lds); break;
    case F_A4G64: prefill_body<Fmt<MOE_W_ASYM, 4, 64>>(a, t, ex, lds); break;
    case F_A4G128: prefill_body<Fmt<MOE_W_ASYM, 4, 128>>(a, t, ex, lds); break;
    case F_A2G16: prefill_body<Fmt<MOE_W_ASYM, 2, 16>>(a, t, ex, lds); break;
    case F_A2G32: prefill_body<Fmt<MOE_W_ASYM, 2, 32>>(a, t, ex, lds); break;
    case F_A2G64: prefill_body<Fmt<MOE_W_ASYM, 2, 64>>(a, t, ex, lds); break;
    case F_A2G128: prefill_body<Fmt<MOE_W_ASYM, 2, 128>>(a, t, ex, lds); break;
    case F_E4G16: prefill_body<Fmt<MOE_W_E2M1, 4, 16>>(a, t, ex, lds); break;
    case F_E4G32: prefill_body<Fmt<MOE_W_E2M1, 4, 32>>(a, t, ex, lds); break;
    case F_E4G64: prefill_body<Fmt<MOE_W_E2M1, 4, 64>>(a, t, ex, lds); break;
    case F_E4G128: prefill_body<Fmt<MOE_W_E2M1, 4, 128>>(a, t, ex, lds); break;
    default: break;
  }
}

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

// one block per token; out[t] = sum_j w[t,j] * sum_s yp[s][inv[t*k+j]]
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ yp, int splits,
                                                         size_t split_stride,
                                                         const float* __restrict__ w,
                                                         const int32_t* __restrict__ inv, int H,
                                                         int k, void* __restrict__ out, int out_dt) {
  const int t = blockIdx.x;
  for (int c4 = threadIdx.x; c4 < H / 4; c4 += kThreads) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = inv[(size_t)t * k + j];
      if (r < 0) continue;  // dropped assignment (out-of-range expert id)
      const float wt = w[(size_t)t * k + j];
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q < splits; ++q)
        y += *reinterpret_cast<const f32x4*>(yp + q * split_stride + (size_t)r * H + 4 * c4);
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
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

inline int max_tiles(int R, int E, int BM) {
  long t = (R + BM - 1) / BM + (R < E ? R : E);
  return (int)t;
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

static hipError_t launch_ffn(FfnArgs& a, int T, int k, bool decode, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  if (decode) {
    const int NB = a.gu ? a.N / 32 : a.N / 64;
    dim3 grid(max_tiles(a.R, a.E, 32) * NB, a.gu ? 1 : a.splits);
    hipLaunchKernelGGL(ffn_decode_kernel, grid, dim3(kThreads), 0, s, a);
  } else {
    const int NB = a.gu ? a.N / 128 : (a.N + 255) / 256;
    dim3 grid(max_tiles(a.R, a.E, kBM) * NB);
    hipLaunchKernelGGL(ffn_prefill_kernel, grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_gate_up(const moe_packed_expert* experts, const int32_t* offsets, int T,
                              int H, int I, int E, int k, const f16* a16, const float* ascale,
                              void* h, int h_f32, bool decode, hipStream_t s) {
  FfnArgs a;
  a.experts = experts;
  a.offsets = offsets;
  a.E = E;
  a.K = H;
  a.N = I;
  a.gu = 1;
  a.a = a16;
  a.ascale = ascale;
  a.out = h;
  a.out_f32 = h_f32;
  a.R = T * k;
  a.splits = 1;
  return launch_ffn(a, T, k, decode, s);
}

hipError_t launch_ffn_down(const moe_packed_expert* experts, const int32_t* offsets, int T,
                           int H, int I, int E, int k, const f16* ain, const float* ascale,
                           float* yp, int splits, bool decode, hipStream_t s) {
  FfnArgs a;
  a.experts = experts;
  a.offsets = offsets;
  a.E = E;
  a.K = I;
  a.N = H;
  a.gu = 0;
  a.a = ain;
  a.ascale = ascale;
  a.out = yp;
  a.out_f32 = 1;
  a.R = T * k;
  a.splits = decode ? splits : 1;
  return launch_ffn(a, T, k, decode, s);
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
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(kThreads), 0, s, yp, splits, stride, w, inv, H,
                     k, out, out_dt);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moeq
