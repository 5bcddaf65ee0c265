// Certified router for prefill batches.
//
// What it computes is the router of the Baidu Cloud article on quantized MoE
// LLM inference ("expert routing" section: router linear, keep the k largest
// logits, softmax over those k): the same ids and weights as the fp64 router
// in route.hip, with far less fp64 work. The mixed-precision field notes
// (section 2.1) keep the router out of low precision because neighbouring
// experts' logits can sit close together; here low precision only proposes,
// and every decision that counts is taken on fp64 values.
//
// Step 0 (cert_prep_kernel): each fp32 router weight is split into two bf16
// numbers, w = wh + wm + r with |r| <= 2^-16 |w| (round-to-nearest
// conversions), stored as two planes, and each router row's fp64 norm is
// taken.
//
// Step 1 (cert_logits_kernel): approximate logits A[t,e] on the bf16 matrix
// cores from those planes; fp32 token rows are split the same way in
// registers, bf16 token rows are exact. The products of bf16 numbers are
// exact in fp32; the 32x32x16 bf16 instruction adds them into an fp32 tile,
// and every kFlush stages (kFlush * 64 columns) the tile is added into fp64
// and restarted from zero. The blocks of the first expert tile also leave
// the fp64 sums of squares of the token rows they stream.
//
// Step 2 (cert_select_kernel, one wavefront per token): an error bound
//   |A[t,e] - L[t,e]| <= d[t,e] = cb * |x_t| |w_e| + 2^-40 |A[t,e]| + tiny,
// with L the exact logit. Its pieces: an fp32 sum of n terms with n - 1
// roundings is off by at most (n - 1) 2^-23 times the sum of the terms'
// magnitudes (any rounding mode that is faithful), the split residuals, the
// fp32 partial stores and the fp64 sums; the magnitudes sum to at most
// |x_t| |w_e| (Cauchy-Schwarz); cb doubles the total as a safety margin, and
// the absolute term covers subnormals flushed to zero. The threshold is the
// k-th largest of the 64 lanes' largest lower ends A - d, which is at most
// the k-th largest lower end: an expert whose upper end A + d lies below it
// has k experts surely above it and is out. The rest (the k winners and any
// expert the bound cannot separate from them, k + 0.1 to 0.5 per token on
// the workloads' inputs) get their logit recomputed exactly as the fp64
// router does, a fixed-order fp64 dot product, and the top-k and the
// softmax run on those values with the fp64 router's tie rule. A token whose
// approximate logits or bounds are not finite (NaN or Inf in x, Wr or b, an
// fp32 overflow) has every expert recomputed, so NaN routing is detected
// exactly as there.
#include "deq.h"
#include "profile.h"
#include "route_dev.h"

namespace moeq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kFlush = 4;                        // stages per fp32 run
constexpr int kSelWaves = 4;                     // tokens per selection block

// 16 bytes per lane from r at voff + soff into LDS at lds + 16 lane
__device__ inline void dma16(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

__device__ inline uint32_t pk_bf16(float a, float b) {
  const bf16x2 p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// 4 fp32 values to their bf16 leading parts and bf16 remainders
__device__ inline void split4(const f32x4 v, u32x2& hi, u32x2& mid) {
  hi[0] = pk_bf16(v[0], v[1]);
  hi[1] = pk_bf16(v[2], v[3]);
  const float r0 = v[0] - __uint_as_float(hi[0] << 16);
  const float r1 = v[1] - __uint_as_float(hi[0] & 0xffff0000u);
  const float r2 = v[2] - __uint_as_float(hi[1] << 16);
  const float r3 = v[3] - __uint_as_float(hi[1] & 0xffff0000u);
  mid[0] = pk_bf16(r0, r1);
  mid[1] = pk_bf16(r2, r3);
}

__device__ inline double sq_bf16x8(const u32x4 v) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double a = (double)__uint_as_float(v[i] << 16);
    const double b = (double)__uint_as_float(v[i] & 0xffff0000u);
    s += a * a + b * b;
  }
  return s;
}
__device__ inline double sq_f32x4(const f32x4 v) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += (double)v[i] * (double)v[i];
  return s;
}

// Router weights to the two bf16 planes the logits kernel multiplies, [2][E][HP]
// (leading parts, then remainders; columns past H zero), and each row's
// fp64 norm. One block per expert row.
__global__ __launch_bounds__(256) void cert_prep_kernel(const float* __restrict__ Wr, int E, int H,
                                                        int HP, uint16_t* __restrict__ Wp,
                                                        double* __restrict__ nw) {
  __shared__ double red[4];
  const int e = blockIdx.x, th = threadIdx.x;
  double acc = 0.0;
  for (int c = 4 * th; c < HP; c += 1024) {
    const f32x4 v = c < H ? *(const f32x4*)(Wr + (size_t)e * H + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    acc += sq_f32x4(v);
    u32x2 hi, mid;
    split4(v, hi, mid);
    *(u32x2*)(Wp + (size_t)e * HP + c) = hi;
    *(u32x2*)(Wp + ((size_t)E + e) * HP + c) = mid;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if ((th & 63) == 0) red[th >> 6] = acc;
  __syncthreads();
  if (th == 0) nw[e] = sqrt(((red[0] + red[1]) + red[2]) + red[3]);
}

// LDS stage of the logits kernel: the token tile (128 rows; bf16: 128 B a
// row, fp32: 256 B), then the two weight planes (BN rows of 128 B each).
// Each row's 16-byte slots hold its column groups XOR-swizzled by the row:
// 128-byte rows take slot = group ^ ((r >> 1) & 7) (rows 2i and 2i+1 sit in
// opposite bank halves of the 64 banks), 256-byte rows slot = group ^ (r & 15);
// the 16 lanes that one matrix-operand read serves at a time then hit 16
// different slots.
template <bool XF, int BN>
struct Lay {
  static constexpr int NW = (kCertTileM / 32) * (BN / 32);  // wavefronts
  static constexpr int NT = 64 * NW;                        // threads
  static constexpr int XB = kCertTileM * (XF ? 256 : 128);  // token tile bytes
  static constexpr int WP = BN * 128;                       // one weight plane
  static constexpr int SB = XB + 2 * WP;                    // stage bytes
  static constexpr int XPARTS = XB / 1024, PARTS = SB / 1024;
  static constexpr int PPW = PARTS / NW;                    // 1 KiB copies per wavefront
  static constexpr int GPR = XF ? 16 : 8;                   // 16-byte groups per token row
  static constexpr int NU = kCertTileM * GPR / NT;          // norm groups per thread
  static_assert(PARTS % NW == 0 && (kCertTileM * GPR) % NT == 0, "stage split");
};
__device__ inline int slot128(int r, int g) { return r * 128 + ((g ^ ((r >> 1) & 7)) << 4); }
__device__ inline int slot256(int r, int g) { return r * 256 + ((g ^ (r & 15)) << 4); }

// One block: 128 tokens x BN experts over the hidden-column chunks
// [kz * cpb, ...) of its K split. Its wavefronts own 32x32 output tiles
// (wave % 4: token quarter, wave / 4: 32-expert slice). Three LDS stages
// filled by direct buffer-to-LDS copies, two chunks ahead of the matrix
// instructions.
template <int XDT, int BN>
__global__ __launch_bounds__(8 * BN) void cert_logits_kernel(
    const void* __restrict__ x, const uint16_t* __restrict__ Wp, int T, int H, int HP, int E,
    int TT, int ET, int KS, int CPB, float* __restrict__ Ap, double* __restrict__ nx2) {
  constexpr bool XF = XDT != MOE_BF16;
  using L = Lay<XF, BN>;
  static_assert(L::NT == 8 * BN, "launch bounds");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[L::SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[L::SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[L::SB];
  // Blocks that share a token tile (and read its x rows) are launched on one
  // XCD: block b runs on XCD b % 8, and takes tile b % 8 * per + b / 8.
  const int nb = TT * ET * KS, per = (nb + 7) >> 3;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= nb) return;
  const int et = lin % ET, kz = (lin / ET) % KS, tt = lin / (ET * KS);
  const int t0 = tt * kCertTileM, e0 = et * BN;
  const int NC = (H + kCertChunk - 1) / kCertChunk;
  const int c0 = kz * CPB, c1 = min(NC, c0 + CPB);
  const int th = threadIdx.x, lane = th & 63;
  const int wave = __builtin_amdgcn_readfirstlane(th >> 6);
  const bool do_nx = et == 0;

  // Copy plan: part p = wave + NW j (j < PPW) of a stage is 1 KiB at byte
  // 1024 p; lane l fills its 16-byte slot l. Per lane: the source offset of
  // its slot (chunk 0), and the same for the last chunk when H is not a
  // multiple of 64 (slots past the row end point past the buffer, which
  // reads as zeros).
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * (XF ? 4 : 2)));
  const rsrc_t rw = make_rsrc(Wp, (uint32_t)((size_t)2 * E * HP * 2));
  uint32_t vo[L::PPW], vt[L::PPW];
  bool isx[L::PPW];
#pragma unroll
  for (int j = 0; j < L::PPW; ++j) {
    const int p = wave + L::NW * j;
    isx[j] = p < L::XPARTS;
    int col, r;
    if (p < L::XPARTS) {
      if (XF) {
        r = 4 * p + (lane >> 4);
        const int g = (lane & 15) ^ (r & 15);
        col = 4 * g;
        vo[j] = (uint32_t)(((size_t)min(t0 + r, T - 1) * H + col) * 4);
      } else {
        r = 8 * p + (lane >> 3);
        const int g = (lane & 7) ^ ((r >> 1) & 7);
        col = 8 * g;
        vo[j] = (uint32_t)(((size_t)min(t0 + r, T - 1) * H + col) * 2);
      }
      const int ct = (NC - 1) * kCertChunk + col;  // column in the last chunk
      vt[j] = ct < H ? vo[j] : 0x80000000u;
    } else {
      const int q = p - L::XPARTS;  // plane q / (BN / 8), rows 8 (q % (BN / 8)) ..
      r = 8 * (q % (BN / 8)) + (lane >> 3);
      const int g = (lane & 7) ^ ((r >> 1) & 7);
      vo[j] = (uint32_t)((((size_t)(q / (BN / 8)) * E + min(e0 + r, E - 1)) * HP + 8 * g) * 2);
      vt[j] = vo[j];
    }
  }
  auto stage = [&](int i) -> uint8_t* { const int m = i % 3; return m == 0 ? st0 : (m == 1 ? st1 : st2); };
  auto issue = [&](int i) {
    const int c = c0 + i;
    const bool tail = c == NC - 1;
    uint8_t* S = stage(i);
#pragma unroll
    for (int j = 0; j < L::PPW; ++j) {
      const int p = wave + L::NW * j;
      const uint32_t soff = isx[j] ? (uint32_t)c * kCertChunk * (XF ? 4 : 2) : (uint32_t)c * kCertChunk * 2;
      dma16(isx[j] ? rx : rw, S + 1024 * p, tail ? vt[j] : vo[j], soff);
    }
  };

  // matrix operands: lane (row ra / rb = its 32-row slice + lane % 32, k half
  // kh = lane / 32); group g = 2 ks + kh of k-step ks
  const int ra = (wave & 3) * 32 + (lane & 31), rb = (wave >> 2) * 32 + (lane & 31);
  const int kh = lane >> 5;
  f32x16 acc = {};
  double a64[16] = {};
  double nxa[L::NU] = {};
  auto compute = [&](const uint8_t* S) {
#pragma unroll
    for (int ks = 0; ks < kCertChunk / 16; ++ks) {
      const int g = 2 * ks + kh;
      const bf16x8 bh = *(const bf16x8*)(S + L::XB + slot128(rb, g));
      const bf16x8 bm = *(const bf16x8*)(S + L::XB + L::WP + slot128(rb, g));
      if constexpr (XF) {
        const f32x4 v0 = *(const f32x4*)(S + slot256(ra, 2 * g));
        const f32x4 v1 = *(const f32x4*)(S + slot256(ra, 2 * g + 1));
        u32x2 h0, m0, h1, m1;
        split4(v0, h0, m0);
        split4(v1, h1, m1);
        const bf16x8 ah = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
        const bf16x8 am = __builtin_bit_cast(bf16x8, u32x4{m0[0], m0[1], m1[0], m1[1]});
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bm, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, bh, acc, 0, 0, 0);
      } else {
        const bf16x8 a = *(const bf16x8*)(S + slot128(ra, g));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bm, acc, 0, 0, 0);
      }
    }
    // squared norms of the token rows (blocks of the first expert tile):
    // group th + NT u of the tile, row (th + NT u) / GPR
    if (do_nx) {
#pragma unroll
      for (int u = 0; u < L::NU; ++u) {
        const int gi = th + L::NT * u, r = gi / L::GPR, g = gi % L::GPR;
        if constexpr (XF)
          nxa[u] += sq_f32x4(*(const f32x4*)(S + slot256(r, g)));
        else
          nxa[u] += sq_bf16x8(*(const u32x4*)(S + slot128(r, g)));
      }
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      a64[r] += (double)acc[r];
      acc[r] = 0.f;
    }
  };

  const int n = c1 - c0;
  if (n > 0) issue(0);
  if (n > 1) issue(1);
  for (int i = 0; i < n; ++i) {
    // chunk i's copies are done once at most the next chunk's are in flight
    if (i + 1 < n)
      __builtin_amdgcn_s_waitcnt(0x0F70 | L::PPW);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // the stage of chunk i + 2 was read in iteration i - 1, before the barrier
    if (i + 2 < n) issue(i + 2);
    compute(stage(i));
    if ((i + 1) % kFlush == 0 || i + 1 == n) flush();
  }

  // partial logits of this K split: lane column e, accumulator rows t
  float* out = Ap + (size_t)kz * T * E;
  const int e = e0 + (wave >> 2) * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + (wave & 3) * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    if (t < T && e < E) out[(size_t)t * E + e] = (float)a64[r];
  }
  if (do_nx) {
    // the GPR threads of a row are consecutive lanes: a fixed butterfly
#pragma unroll
    for (int u = 0; u < L::NU; ++u) {
      double v = nxa[u];
#pragma unroll
      for (int o = 1; o < L::GPR; o <<= 1) v += __shfl_xor(v, o);
      const int gi = th + L::NT * u, t = t0 + gi / L::GPR;
      if (gi % L::GPR == 0 && t < T) nx2[(size_t)kz * T + t] = v;
    }
  }
}

// Token row t in registers, one slice of 512 * NG columns: lane l holds the
// 8-column groups l + 64 g (g < NG), zero past the row end. Buffer loads:
// the row's offset is scalar, a lane's columns past the row end point past
// the buffer (which reads as zeros).
template <int XDT, int NG>
struct XRow {
  static constexpr int XE = XDT == MOE_BF16 ? 2 : 4;  // bytes per element
  u32x4 b[XDT == MOE_BF16 ? NG : 1];
  f32x4 f[XDT == MOE_BF16 ? 1 : 2 * NG];
  int base;  // first column of the slice held
  __device__ inline void load(rsrc_t rx, int H, int t, int s0) {
    const int lane = threadIdx.x & 63;
    base = s0;
    const uint32_t so = (uint32_t)t * H * XE;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int col = s0 + 8 * (lane + 64 * g);
      const uint32_t vo = col < H ? (uint32_t)col * XE : 0x80000000u;
      if (XDT == MOE_BF16) {
        b[g] = bload<u32x4>(rx, vo, so);
      } else {
        f[2 * g] = bload<f32x4>(rx, vo, so);
        f[2 * g + 1] = bload<f32x4>(rx, vo + 16, so);
      }
    }
  }
  // An empty asm that claims to change the registers: keeps the compiler
  // from hoisting the fp64 conversions of the whole slice out of the
  // candidate loop (that would hold 16 NG fp64 registers instead of 4 NG).
  __device__ inline void touch() {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (XDT == MOE_BF16) {
        asm volatile("" : "+v"(b[g]));
      } else {
        asm volatile("" : "+v"(f[2 * g]));
        asm volatile("" : "+v"(f[2 * g + 1]));
      }
    }
  }
  __device__ inline double at(int g, int i) const {
    if (XDT == MOE_BF16)
      return (double)__uint_as_float(i & 1 ? (b[g][i >> 1] & 0xffff0000u) : (b[g][i >> 1] << 16));
    return (double)f[2 * g + (i >> 2)][i & 3];
  }
};

// Sum of v over the wavefront in a fixed order, the same value in every
// lane: pairwise exchanges (lane ^ 1, ^ 2 within quads, the mirrored lane of
// each 8- and 16-lane row, then lane ^ 16 and ^ 32). Each step adds two
// values that both lanes of a pair hold, so the pair stays equal.
__device__ inline double dpp_f64(double v, int ctrl_sel) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  switch (ctrl_sel) {
    case 0:
      lo = __builtin_amdgcn_update_dpp(0, (int)lo, 0xB1, 0xF, 0xF, false);
      hi = __builtin_amdgcn_update_dpp(0, (int)hi, 0xB1, 0xF, 0xF, false);
      break;
    case 1:
      lo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x4E, 0xF, 0xF, false);
      hi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x4E, 0xF, 0xF, false);
      break;
    case 2:  // row_half_mirror
      lo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x141, 0xF, 0xF, false);
      hi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x141, 0xF, 0xF, false);
      break;
    default:  // row_mirror
      lo = __builtin_amdgcn_update_dpp(0, (int)lo, 0x140, 0xF, 0xF, false);
      hi = __builtin_amdgcn_update_dpp(0, (int)hi, 0x140, 0xF, 0xF, false);
      break;
  }
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ inline double dpp_bcast_f64(double v, int ctrl, int row_mask) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t lo, hi;
  if (ctrl == 0x142) {
    lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x142, 0xA, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x142, 0xA, 0xF, false);
  } else {
    lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x143, 0xC, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x143, 0xC, 0xF, false);
  }
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Row sums as above, then row 1 adds row 0's and row 3 row 2's (lane 15
// broadcast), row 3 adds row 1's (lane 31 broadcast): lane 63 holds
// ((R2 + R3) + (R0 + R1)), read into a scalar register.
__device__ inline double wave_sum_f64(double v) {
  v += dpp_f64(v, 0);
  v += dpp_f64(v, 1);
  v += dpp_f64(v, 2);
  v += dpp_f64(v, 3);
  v += dpp_bcast_f64(v, 0x142, 0xA);  // rows 0 and 2 add the zero the copy leaves them
  v += dpp_bcast_f64(v, 0x143, 0xC);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Exact fp64 dot products of token row t with router rows e0 and (nb == 2)
// e1, both wave-uniform: x slices come from xr (slice 0 preloaded), router
// columns in batches of 4 groups per lane with all their loads issued before
// the multiplies.
template <int XDT, int NG>
__device__ inline void exact_dots(rsrc_t rx, rsrc_t rw, int H, int t, XRow<XDT, NG>& xr, int e0,
                                  int e1, int nb, double& s0, double& s1) {
  constexpr int GQ = NG < 4 ? NG : 4;
  const int lane = threadIdx.x & 63;
  s0 = 0.0;
  s1 = 0.0;
  xr.touch();
  const uint32_t so0 = (uint32_t)e0 * H * 4, so1 = (uint32_t)e1 * H * 4;
  for (int c0 = 0; c0 < H; c0 += 512 * NG) {
    if (xr.base != c0) xr.load(rx, H, t, c0);
#pragma unroll
    for (int q = 0; q < NG; q += GQ) {
      f32x4 w0[GQ][2], w1[GQ][2];
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        const int col = c0 + 8 * (lane + 64 * (q + g));
        const uint32_t vo = col < H ? (uint32_t)col * 4 : 0x80000000u;
        w0[g][0] = bload<f32x4>(rw, vo, so0);
        w0[g][1] = bload<f32x4>(rw, vo + 16, so0);
        if (nb == 2) {
          w1[g][0] = bload<f32x4>(rw, vo, so1);
          w1[g][1] = bload<f32x4>(rw, vo + 16, so1);
        } else {
          w1[g][0] = f32x4{0.f, 0.f, 0.f, 0.f};
          w1[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int g = 0; g < GQ; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double xv = xr.at(q + g, i);
          s0 += xv * (double)w0[g][i >> 2][i & 3];
          s1 += xv * (double)w1[g][i >> 2][i & 3];
        }
    }
  }
  s0 = wave_sum_f64(s0);
  s1 = wave_sum_f64(s1);
}

// k rounds of a wave-wide argmax over the live slots v[j] (expert lane +
// 64 j), ties to the lower expert: lane r < k receives the r-th value and
// expert; last_v (every lane) the k-th value.
__device__ inline void topk_rounds(const double (&v)[4], const bool (&live)[4], int k,
                                   double& my_v, int& my_i, double& top_v, double& last_v) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
    double best_v = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t key = (live[j] && !((taken >> j) & 1u)) ? rt::order_key(v[j], lane + 64 * j) : 0ull;
      if (key > best) {
        best = key;
        best_v = v[j];
      }
    }
    const uint64_t win = rt::wave_max_u64(best);
    const int wi = 255 - (int)(win & 0xFF);
    const double wv = __shfl(best_v, wi & 63);
    if (r == 0) top_v = wv;
    last_v = wv;
    if (lane == r) {
      my_v = wv;
      my_i = wi;
    }
    if ((wi & 63) == lane) taken |= 1u << (wi >> 6);
  }
}

// fp32 at or below v (v not NaN)
__device__ inline float f32_down(double v) {
  float f = (float)v;
  if ((double)f > v) {
    const uint32_t u = __float_as_uint(f);
    f = f > 0.f ? __uint_as_float(u - 1) : (f == 0.f ? __uint_as_float(0x80000001u) : __uint_as_float(u + 1));
  }
  return f;
}
// fp32 bits made monotone as unsigned integers
__device__ inline uint32_t f32_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_f32(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7fffffffu) : ~k);
}
// maximum over the wavefront, read into a scalar register: row maxima by
// DPP, then the lane 15 / lane 31 broadcasts carry them into row 3
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

template <int XDT, int NG>
__global__ __launch_bounds__(64 * kSelWaves) void cert_select_kernel(
    const void* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias, int T,
    int H, int E, int k, int KS, const float* __restrict__ Ap, const double* __restrict__ nx2,
    const double* __restrict__ nwv, double cb, int32_t* __restrict__ ids, float* __restrict__ w) {
  // the token index in a scalar register (buffer offsets derived from it
  // must be known to be wavefront-uniform)
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * kSelWaves + threadIdx.x / 64);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * XRow<XDT, NG>::XE));
  const rsrc_t rw = make_rsrc(Wr, (uint32_t)((size_t)E * H * 4));
  XRow<XDT, NG> xr;
  xr.load(rx, H, t, 0);  // in flight while the bounds are worked out
  double nxs = 0.0;
  for (int q = 0; q < KS; ++q) nxs += nx2[(size_t)q * T + t];
  const double nx = sqrt(nxs);
  const double sqh = sqrt((double)H);
  // approximate logits and their bounds
  double A[4], D[4];
  bool valid[4];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < E;
    const int ec = min(e, E - 1);
    double a = 0.0;
    for (int q = 0; q < KS; ++q) a += (double)Ap[((size_t)q * T + t) * E + ec];
    if (bias) a += (double)bias[ec];
    const double nw = nwv[ec];
    const double d = cb * nx * nw + 0x1p-40 * fabs(a) + 0x1p-120 * ((double)H + sqh * (nx + nw));
    A[j] = a;
    D[j] = d;
    bad |= valid[j] && !(__builtin_isfinite(a) && __builtin_isfinite(d));
  }
  bad = __any(bad);
  bool cand[4];
  if (!bad) {
    // A threshold at or below the k-th largest lower end A - d: the k-th
    // largest of the lanes' own largest lower ends (in fp32, rounded down).
    // Experts whose upper end falls below it are out.
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (valid[j]) m = fmaxf(m, f32_down(A[j] - D[j]));
    uint32_t key = f32_key(m), kth = 0;
    for (int r = 0; r < k; ++r) {
      kth = wave_max_u32(key);
      const uint64_t own = __ballot(key == kth);
      if (lane == __builtin_ctzll(own)) key = 0;  // remove one holder of the maximum
    }
    const double tau = (double)key_f32(kth);
#pragma unroll
    for (int j = 0; j < 4; ++j) cand[j] = valid[j] && A[j] + D[j] >= tau;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) cand[j] = valid[j];
  }
  // exact logits of the candidates, two at a time, in expert order: the
  // owner lane's slot X[j] gets each, and lane i the i-th candidate
  // (value cv, expert ce) while there are at most 64
  uint64_t mk[4];
  int nc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mk[j] = __ballot(cand[j]);
    nc += __builtin_popcountll(mk[j]);
  }
  double X[4] = {0.0, 0.0, 0.0, 0.0};
  double cv = 0.0;
  int ce = 0, ci = 0, jj = 0;
  while (true) {
    int eb[2] = {0, 0};
    int nb = 0;
    while (nb < 2 && jj < 4) {
      if (mk[jj]) {
        const int b = __builtin_ctzll(mk[jj]);
        mk[jj] &= mk[jj] - 1;
        eb[nb++] = 64 * jj + b;
      } else {
        ++jj;
      }
    }
    if (nb == 0) break;
    double s[2];
    exact_dots<XDT, NG>(rx, rw, H, t, xr, eb[0], nb == 2 ? eb[1] : eb[0], nb, s[0], s[1]);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b < nb) {
        const double v = s[b] + (bias ? (double)bias[eb[b]] : 0.0);
        if (lane == (eb[b] & 63)) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j == (eb[b] >> 6)) X[j] = v;
        }
        if (lane == ci + b) {
          cv = v;
          ce = eb[b];
        }
      }
    }
    ci += nb;
  }
  if (nc <= 64) {
    // rank of candidate i = number of candidates ahead of it (larger value,
    // or equal value and lower expert: the fp64 router's order key)
    const bool live = lane < nc;
    const uint64_t key = live ? rt::order_key(cv, ce) : 0ull;
    const bool nan_row = __any(live && cv != cv);
    int rank = 0;
    for (int j = 0; j < nc; ++j) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)key, j);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(key >> 32), j);
      rank += (((uint64_t)hi << 32) | lo) > key;
    }
    const bool sel = live && rank < k;
    const uint64_t first = __ballot(sel && rank == 0);
    const double top_v = __shfl(cv, __builtin_ctzll(first));
    const double ex = sel ? exp(cv - top_v) : 0.0;
    double den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (sel) {
      ids[(size_t)t * k + rank] = nan_row ? MOE_ID_NAN : ce;
      w[(size_t)t * k + rank] = nan_row ? 0.f : (float)(ex / den);
    }
    return;
  }
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) nan_seen |= cand[j] && X[j] != X[j];
  const bool nan_row = __any(nan_seen);
  double my_v = 0.0, top_v = 0.0, last_v;
  int my_i = 0;
  topk_rounds(X, cand, k, my_v, my_i, top_v, last_v);
  const double ex = lane < k ? exp(my_v - top_v) : 0.0;
  double den = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = nan_row ? MOE_ID_NAN : my_i;
    w[(size_t)t * k + lane] = nan_row ? 0.f : (float)(ex / den);
  }
}

// cb of the bound for token dtype XDT, K splits ks and H columns
double cert_cb(int xdt, int ks, int H) {
  const double n = (double)kFlush * kCertChunk * (xdt == MOE_BF16 ? 2 : 3);  // terms per fp32 run
  const double run = 1.02 * (n - 1.0) * 0x1p-23;  // roundings of one run, per unit of magnitude
  const double split = xdt == MOE_BF16 ? 0x1p-16 : 3.1 * 0x1p-16;  // dropped split terms
  const double rest = 0x1p-23 + ((double)H / kCertChunk + ks + 2.0) * 0x1p-52;  // stores, fp64 sums
  return 2.0 * (run + split + rest);
}

template <int XDT>
hipError_t launch_cert_x(const void* x, const float* Wr, const float* b, int T, int H, int E,
                         int k, int32_t* ids, float* w, void* ws, const CertPlan& p,
                         hipStream_t s) {
  uint8_t* base = (uint8_t*)ws;
  float* Ap = (float*)(base + p.ap);
  double* nx2 = (double*)(base + p.nx);
  double* nw = (double*)(base + p.nw);
  uint16_t* Wp = (uint16_t*)(base + p.wp);
  hipLaunchKernelGGL(cert_prep_kernel, dim3(E), dim3(256), 0, s, Wr, E, H, p.hp, Wp, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = p.tt * p.et * p.ks;
  const int grid = ((nb + 7) >> 3) * 8;
  // (128-expert tiles with fp32 token rows would not fit the LDS; the plan
  // never asks for them)
  if constexpr (XDT == MOE_BF16)
    if (p.bn == 128) {
      hipLaunchKernelGGL((cert_logits_kernel<XDT, 128>), dim3(grid),
                         dim3(Lay<XDT != MOE_BF16, 128>::NT), 0, s, x, Wp, T, H, p.hp, E, p.tt,
                         p.et, p.ks, p.cpb, Ap, nx2);
    }
  if (XDT != MOE_BF16 || p.bn != 128)
    hipLaunchKernelGGL((cert_logits_kernel<XDT, 64>), dim3(grid),
                       dim3(Lay<XDT != MOE_BF16, 64>::NT), 0, s, x, Wp, T, H, p.hp, E, p.tt,
                       p.et, p.ks, p.cpb, Ap, nx2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int sel = (T + kSelWaves - 1) / kSelWaves;
  const double cb = cert_cb(XDT, p.ks, H);
  // slice of the token row held in registers: 512 * NG columns (wider rows
  // take several slices)
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(sel), dim3(64 * kSelWaves), 0, s, x, Wr, b, T, H, E, k, p.ks,
                       Ap, nx2, nw, cb, ids, w);
  };
  if (H <= 1024)
    go(cert_select_kernel<XDT, 2>);
  else
    go(cert_select_kernel<XDT, 4>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_cert(const void* x, int xdt, const float* Wr, const float* b, int T,
                             int H, int E, int k, int32_t* ids, float* w, void* ws,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const CertPlan p = cert_plan(T, H, E, xdt);
  if (!p.use) return hipErrorInvalidValue;
  return xdt == MOE_BF16 ? launch_cert_x<MOE_BF16>(x, Wr, b, T, H, E, k, ids, w, ws, p, s)
                         : launch_cert_x<MOE_F32>(x, Wr, b, T, H, E, k, ids, w, ws, p, s);
}

}  // namespace moeq
