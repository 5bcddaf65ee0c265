// int8 prefill GEMM for 4-bit asymmetric weights and int8 activations
// (W4A8: the MoE mixed-precision notes' per-token int8 expert inputs,
// section 2.1, on the "AlphaQ" blog's group-wise 4-bit weights, section 4.2).
//
// With asymmetric weights w = s_g q + m_g (per weight row and group g of GE
// columns) and int8 codes a of a token row, a row's dot product is
//   sum_g ( s_g * sum_{k in g} a_k q_k  +  m_g * sum_{k in g} a_k ).
// The inner sums are integers: the 4-bit codes unpack to bytes and go
// through v_mfma_i32_32x32x32_i8 exactly, each group's int32 accumulators
// start from zero, and at the end of a group they are converted and scaled
// into fp32 accumulators together with the minimum times the rows' code sum
// (the 64-column sums come precomputed with the codes). The row scale of the
// int8 codes is applied in the epilogue, as in the fp16 kernels.
//
// Operand order: a weight word holds 8 consecutive codes with code 2i in
// nibble i and code 2i+1 in nibble i+4; masking the even and the odd
// nibbles gives bytes in the order 0,4,1,5,2,6,3,7 ("perm8"). The token
// codes are stored in that order (store8_i8p), so both operands of every
// MFMA list the same k in the same byte position.
//
// Block: 128 token rows x 4 units (GU: 32 outputs = 32 gate + 32 up rows;
// DN: 64 outputs), 8 wavefronts = 2 row halves x 4 units, one block per CU
// (two wavefronts per SIMD). K tiles of 128: the token tile (16 KiB of codes)
// and its row sums reach LDS by DMA, double-buffered; each wavefront streams
// its two weight row tiles into registers two tiles ahead.
#pragma once

#include "gemm_impl.h"

namespace moeq {

// The int8 GEMM of format fid (F_A4G128) in role R_GU or R_DN on a.a8 /
// a.asum (hipErrorNotSupported for any other format or role).
hipError_t launch_ffn_i8(int fid, int role, const FfnArgs& a, hipStream_t s);

namespace {

constexpr int kI8W = 8;     // wavefronts per block
constexpr int kI8KT = 128;  // K tile: codes per token row

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// one K tile's weights of a wavefront: its two row tiles' codes (the packed
// 4-bit tiles 2kt and 2kt+1, 16 bytes per lane each) and their parameters
// (fp16 scale in the low half, fp16 minimum in the high half)
template <int GE>
struct I8Tile {
  u32x4 c[2][2];
  uint32_t p[2][kI8KT / GE];
};

template <int ROLE, int GE>
__global__ __launch_bounds__(64 * kI8W, 1) void ffn_prefill_i8_kernel(FfnArgs a) {
  using F = Fmt<MOE_W_ASYM, 4, GE>;
  // groups of 64 would fit the step layout too, but their kernel spills
  static_assert(GE == 128, "groups of 128 columns");
  constexpr bool GU = ROLE == R_GU;
  constexpr int NGT = kI8KT / GE;               // weight groups per K tile
  constexpr int TILEB = kBM * kI8KT;            // 16 KiB
  constexpr int NI = TILEB / (kI8W * 64 * 16);  // DMA instructions per wavefront and tile
  static_assert(NI * kI8W * 64 * 16 == TILEB, "token tile DMA");
  constexpr int LPT = 4 + 2 * NGT;              // weight loads per wavefront and tile
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[TILEB];
  // the tile's 64-column code sums, [row][2] (rows of the block)
  __shared__ __attribute__((aligned(16))) float sm0[kBM * 2];
  __shared__ __attribute__((aligned(16))) float sm1[kBM * 2];
  const int NU = a.N / (GU ? 32 : 64);
  const int NB = (NU + 3) / 4;
  Task t;
  if (!find_task_lpt<ROLE>(a, F::ID, kBM, NB, blockIdx.x, t)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kh = lane >> 5;
  const int mh = wave & 1, uw = wave >> 1;
  const int KTn = a.K / kI8KT, KT4 = a.K / 64, NE = a.K / GE;
  const moe_packed_expert* ex = a.experts + t.e;
  const uint8_t *codes, *params;
  role_matrix<ROLE>(ex, codes, params);
  const int unit = 4 * t.nt + uw;
  const bool on = unit < NU;
  const int rtl = 2 * min(unit, NU - 1);
  const int NRT = GU ? 2 * a.N / 32 : a.N / 32;
  const rsrc_t rC = make_rsrc(uniform_ptr(codes), (uint32_t)((size_t)NRT * KT4 * 1024));
  const rsrc_t rP = make_rsrc(uniform_ptr(params), (uint32_t)((size_t)NRT * NE * 32 * 4));
  const rsrc_t rA = make_rsrc(a.a8, (uint32_t)((size_t)a.R * a.K));
  const rsrc_t rS = make_rsrc(a.asum, (uint32_t)((size_t)a.R * (a.K / 64) * 4));
  const uint32_t vc0 = (uint32_t)rtl * KT4 * 1024 + lane * 16;
  const uint32_t vc1 = vc0 + (uint32_t)KT4 * 1024;
  const uint32_t vp0 = ((uint32_t)rtl * NE * 32 + n) * 4;
  const uint32_t vp1 = vp0 + (uint32_t)NE * 32 * 4;

  // Token tile DMA: 128 rows x 8 chunks of 16 bytes, chunk c of row r stored
  // at c ^ swz(r); rows past the segment repeat its last row. Wavefront 0
  // also brings the tile's row sums (2 rows per lane; rows past the segment
  // are other rows' sums, and their outputs are never stored).
  auto swz = [](int r) { return (r >> 1) & 7; };
  uint32_t doff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int slot = (wave * NI + j) * 64 + lane;
    const int r = slot >> 3, c = (slot & 7) ^ swz(slot >> 3);
    doff[j] = (uint32_t)((size_t)(t.row0 + min(r, t.mcount - 1)) * a.K + 16 * c);
  }
  const uint32_t soff = (uint32_t)(t.row0 + 2 * lane) * 8;
  const uint32_t sstride = (uint32_t)a.R * 8;  // bytes of one K tile's sums
  auto dma = [&](int kt, uint8_t* buf, float* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      dma16(rA, buf + (wave * NI + j) * 1024, doff[j], (uint32_t)kt * kI8KT);
    if (wave == 0) dma16(rS, reinterpret_cast<uint8_t*>(sb), soff, (uint32_t)kt * sstride);
  };
  auto load_w = [&](int kt, I8Tile<GE>& w) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)(2 * kt) * 1024;
    w.c[0][0] = bload<u32x4>(rC, vc0, so);
    w.c[0][1] = bload<u32x4>(rC, vc0, so + 1024);
    w.c[1][0] = bload<u32x4>(rC, vc1, so);
    w.c[1][1] = bload<u32x4>(rC, vc1, so + 1024);
#pragma unroll
    for (int g = 0; g < NGT; ++g) {
      const uint32_t sp = (uint32_t)(kt * NGT + g) * 32 * 4;
      w.p[0][g] = bload<uint32_t>(rP, vp0, sp);
      w.p[1][g] = bload<uint32_t>(rP, vp1, sp);
    }
  };
  // filled 32-row sub-tiles of this wavefront's half (block-uniform per half)
  const int amt = __builtin_amdgcn_readfirstlane((t.mcount + 31) / 32);
  const int aw = min(max(amt - 2 * mh, 0), 2);

  f32x16 accf[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    accf[mi][0] = f32x16{};
    accf[mi][1] = f32x16{};
  }
  auto run = [&](auto aw_c) __attribute__((always_inline)) {
    constexpr int AW = decltype(aw_c)::value;
    // one K tile: 4 MFMA steps of 32 columns; step s covers, for lane half
    // kh, columns 64 (s / 2) + 32 kh + 16 (s % 2) + [0, 16) of the tile
    auto compute = [&](const uint8_t* buf, const float* sb, const I8Tile<GE>& w) __attribute__((always_inline)) {
      if constexpr (AW > 0) {
        i32x16 acc[AW][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          i32x4 av[AW];
#pragma unroll
          for (int mi = 0; mi < AW; ++mi) {
            const int c = (4 * (s >> 1) + 2 * kh + (s & 1)) ^ swz(n);
            av[mi] = *reinterpret_cast<const i32x4*>(buf + ((2 * mh + mi) * 32 + n) * kI8KT + c * 16);
          }
          i32x4 b[2];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const uint32_t w0 = w.c[tt][s >> 1][2 * (s & 1)], w1 = w.c[tt][s >> 1][2 * (s & 1) + 1];
            b[tt] = i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                          (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
          }
          // a group's first step starts from zero
          const bool first = GE == 64 ? (s & 1) == 0 : s == 0;
#pragma unroll
          for (int mi = 0; mi < AW; ++mi) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
              acc[mi][tt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                  av[mi], b[tt], first ? i32x16{} : acc[mi][tt], 0, 0, 0);
          }
          // end of a group: scale the integer sums into fp32
          const bool last = GE == 64 ? (s & 1) == 1 : s == 3;
          if (last) {
            const int g = GE == 64 ? s >> 1 : 0;
            float sc[2], mn[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const uint32_t p = w.p[tt][g];
              sc[tt] = (float)__builtin_bit_cast(f16, (uint16_t)(p & 0xffffu));
              mn[tt] = (float)__builtin_bit_cast(f16, (uint16_t)(p >> 16));
            }
#pragma unroll
            for (int mi = 0; mi < AW; ++mi) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                // one row quad at a time: the sums are read where used
                __builtin_amdgcn_sched_barrier(0);
                // rows 8q + 4kh + 0..3 of the sub-tile: their two 64-column sums
                const int row = (2 * mh + mi) * 32 + 8 * q + 4 * kh;
                const f32x4 s01 = *reinterpret_cast<const f32x4*>(sb + row * 2);
                const f32x4 s23 = *reinterpret_cast<const f32x4*>(sb + row * 2 + 4);
                float as[4];
                if constexpr (GE == 128) {
                  as[0] = s01[0] + s01[1];
                  as[1] = s01[2] + s01[3];
                  as[2] = s23[0] + s23[1];
                  as[3] = s23[2] + s23[3];
                } else {
                  as[0] = s01[g];
                  as[1] = s01[2 + g];
                  as[2] = s23[g];
                  as[3] = s23[2 + g];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int r = 4 * q + i;
#pragma unroll
                  for (int tt = 0; tt < 2; ++tt)
                    accf[mi][tt][r] = fmaf(sc[tt], (float)acc[mi][tt][r],
                                           fmaf(mn[tt], as[i], accf[mi][tt][r]));
                }
              }
            }
          }
          // one scheduling region per step
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // Pipeline, one barrier per K tile, two token buffers and two weight
    // slots: tile kt issues the DMA of token tile kt+1 after its barrier
    // (into the buffers tile kt-1 used) and, after its MFMAs, the weights of
    // tile kt+2 into the slot it used. At its start the weights of tile kt
    // (issued after the DMA of tile kt) must have landed, so only the
    // weights of tile kt+1 stay in flight. Prefetches past the last tile
    // re-read the last tile (unused). (Three buffers unrolled over six tiles
    // spilled: the scheduler mixed the tiles.)
    I8Tile<GE> W0, W1;
    // a wavefront without rows never reads its weight slots, so the compiler
    // drops their loads: it then waits for all of its memory operations (its
    // DMA of tile kt is the last it issued before the barrier of tile kt)
    constexpr int VM = AW == 0 ? 0 : LPT;
    auto tile = [&](int kt, uint8_t* cur, float* scur, uint8_t* nx, float* snx,
                    I8Tile<GE>& slot) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70 | (VM & 15) | ((VM >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      dma(min(kt + 1, KTn - 1), nx, snx);
      compute(cur, scur, slot);
      load_w(min(kt + 2, KTn - 1), slot);
    };
    load_w(0, W0);
    dma(0, lds0, sm0);
    load_w(min(1, KTn - 1), W1);
    int kt = 0;
    for (; kt + 1 < KTn; kt += 2) {
      tile(kt, lds0, sm0, lds1, sm1, W0);
      tile(kt + 1, lds1, sm1, lds0, sm0, W1);
    }
    if (kt < KTn) tile(kt, lds0, sm0, lds1, sm1, W0);
  };
  if (aw == 2) run(IntC<2>{});
  else if (aw == 1) run(IntC<1>{});
  else run(IntC<0>{});
  // no DMA may still be in flight when the block's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (!on) return;

  // Epilogue, straight from the accumulators: for each register, the 32
  // lanes of a half write 32 consecutive outputs of one row.
  bool over = false;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    if (mi >= aw) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = (2 * mh + mi) * 32 + acc_row(r, lane);
      if (lr >= t.mcount) continue;
      const int row = t.row0 + lr;
      const float sc = a.ascale[row];
      if constexpr (GU) {
        const float h = silu_mul(accf[mi][0][r] * sc, accf[mi][1][r] * sc);
        const size_t o = (size_t)row * a.N + 32 * unit + n;
        if (a.out_f32) {
          reinterpret_cast<float*>(a.out)[o] = h;
        } else {
          reinterpret_cast<f16*>(a.out)[o] = (f16)h;
          over |= fabsf(h) > kF16Max;
        }
      } else {
        float* y = reinterpret_cast<float*>(a.out) + (size_t)row * a.N + 64 * unit + n;
        y[0] = accf[mi][0][r] * sc;
        y[32] = accf[mi][1][r] * sc;
      }
    }
  }
  if (GU && over && a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_FP16_RANGE);
}

template <int ROLE, int GE>
hipError_t launch_i8_one(const FfnArgs& a, hipStream_t s) {
  const int NU = a.N / (ROLE == R_GU ? 32 : 64);
  const int NB = (NU + 3) / 4;
  const long nblk = (long)max_tiles(a.R, a.E, kBM) * NB;
  FfnArgs b = a;
  // one block per CU: expert-major from 4 blocks per CU, else longest first
  b.lpt = nblk < 4L * device_cus() ? 1 : 0;
  // 16 spare blocks: the per-XCD task shares may round up (find_task_lpt)
  hipLaunchKernelGGL((ffn_prefill_i8_kernel<ROLE, GE>), dim3(nblk + 16), dim3(64 * kI8W), 0, s,
                     b);
  return hipGetLastError();
}

}  // namespace
}  // namespace moeq
