// Grouped expert GEMMs: gate/up + SwiGLU and the down projection, on weights
// decoded in registers from packed 4-/3-/2-/1-bit and e2m1 blocks (kernel
// templates; each gemm_<family>.hip instantiates its formats, gemm.hip
// dispatches).
//
// Expert FFN: three matrices per expert, gate/up/down ("AlphaQ" blog,
// section 2.2; MoE mixed-precision notes, section 3.3), in the gated SwiGLU
// form h = silu(a Wg^T) * (a Wu^T), y = h Wd^T. SwiGLU is fused into the
// gate/up epilogue (the notes fuse the expert activation into the linear,
// section 3.6). Only the experts a token was routed to are read ("Sparse
// activation ... 2% activation", section 3.1: the saving is in bandwidth).
//
// Two kernel families share the tile layout and the in-register decoding:
//  * decode (few rows per expert): a block is 4 wavefronts on the same 32-row
//    token tile; they form 4/ksw row groups (64 weight rows each) whose ksw
//    wavefronts split the K tiles, ksw chosen from K so every wavefront
//    streams at least 16 tiles. Weights stream from HBM straight into
//    registers (non-temporal 16-byte loads per lane, 1 KiB per wave and
//    tile, two tiles ahead), are decoded to fp16 and fed to
//    v_mfma_f32_32x32x16_f16 with the token rows padded to 32; partial sums
//    meet in LDS. The down projection also splits K across blocks.
//  * prefill (many rows per expert): a block owns 128 token rows and 4 x 64
//    weight rows; the token tile reaches LDS by DMA (buffer loads with an
//    LDS destination, rows swizzled for the 64-bank LDS, three buffers for
//    4-bit tiles) and is shared by the 4 wavefronts, each of which streams
//    its own weight rows into registers (buffer loads: scalar base and tile
//    offset, so no vector address arithmetic) and decodes step s+1 while the
//    MFMAs of step s run; two
//    blocks share a CU so one block's decode overlaps the other's MFMAs. The
//    pipeline is specialised on the number of 32-row sub-tiles holding rows,
//    so a partial last m-tile costs only its own MFMAs, and each XCD runs
//    its full m-tiles before its partial ones (longest first).
// Every kernel is instantiated per block format; a launch handles the experts
// of its format. Tasks are (expert, n-tile, m-tile), expert-major, so blocks
// that share weight tiles run together; each block derives its task from the
// segment offsets, so no host synchronisation is needed.
#pragma once

#include "common.h"
#include "deq.h"

namespace moeq {

// Arguments of one grouped-GEMM launch (shared by the per-format units).
struct FfnArgs {
  const moe_packed_expert* experts;
  const int32_t* offsets;
  uint32_t* flags;
  uint32_t fmt_mask;
  int E;
  int K;          // reduction dim (H for gate/up, I for down)
  int N;          // outputs per expert (I for gate/up, H for down)
  const f16* a;   // [R, K] rows in sorted order
  const float* ascale;  // per-row scale (int8 inputs) or null
  void* out;      // gate/up: h [R, N] (f16 or f32); down: [splits][R][N] f32
  int out_f32;
  int R;
  int splits;
  int lpt;        // prefill task order: expert-major (0), longest first in 2 (1) or 4 (2) classes
  // prefill outlier corrections: the transposed inputs (see OutlierInputs)
  const f16* at = nullptr;
  int rp = 0;
  const int32_t* poff = nullptr;
  // int8 prefill GEMMs (format F_A4G128): the codes in perm8 order and
  // their 64-column sums (nullptr: the fp16 kernels run)
  const int8_t* a8 = nullptr;
  const float* asum = nullptr;
};

// Launches the grouped GEMM of format `fid` in role `role` (one unit per
// format family: gemm_a4.hip, gemm_a2.hip, gemm_e4.hip, gemm_a1.hip,
// gemm_a3.hip).
hipError_t launch_ffn_fmt(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);

namespace {

constexpr int kThreads = 256;

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int FID>
struct FmtOf;
template <> struct FmtOf<F_A4G16> { using T = Fmt<MOE_W_ASYM, 4, 16>; };
template <> struct FmtOf<F_A4G32> { using T = Fmt<MOE_W_ASYM, 4, 32>; };
template <> struct FmtOf<F_A4G64> { using T = Fmt<MOE_W_ASYM, 4, 64>; };
template <> struct FmtOf<F_A4G128> { using T = Fmt<MOE_W_ASYM, 4, 128>; };
template <> struct FmtOf<F_A2G16> { using T = Fmt<MOE_W_ASYM, 2, 16>; };
template <> struct FmtOf<F_A2G32> { using T = Fmt<MOE_W_ASYM, 2, 32>; };
template <> struct FmtOf<F_A2G64> { using T = Fmt<MOE_W_ASYM, 2, 64>; };
template <> struct FmtOf<F_A2G128> { using T = Fmt<MOE_W_ASYM, 2, 128>; };
template <> struct FmtOf<F_E4G16> { using T = Fmt<MOE_W_E2M1, 4, 16>; };
template <> struct FmtOf<F_E4G32> { using T = Fmt<MOE_W_E2M1, 4, 32>; };
template <> struct FmtOf<F_E4G64> { using T = Fmt<MOE_W_E2M1, 4, 64>; };
template <> struct FmtOf<F_E4G128> { using T = Fmt<MOE_W_E2M1, 4, 128>; };
template <> struct FmtOf<F_A1G16> { using T = Fmt<MOE_W_ASYM, 1, 16>; };
template <> struct FmtOf<F_A1G32> { using T = Fmt<MOE_W_ASYM, 1, 32>; };
template <> struct FmtOf<F_A1G64> { using T = Fmt<MOE_W_ASYM, 1, 64>; };
template <> struct FmtOf<F_A1G128> { using T = Fmt<MOE_W_ASYM, 1, 128>; };
template <> struct FmtOf<F_A3G16> { using T = Fmt<MOE_W_ASYM, 3, 16>; };
template <> struct FmtOf<F_A3G32> { using T = Fmt<MOE_W_ASYM, 3, 32>; };
template <> struct FmtOf<F_A3G64> { using T = Fmt<MOE_W_ASYM, 3, 64>; };
template <> struct FmtOf<F_A3G128> { using T = Fmt<MOE_W_ASYM, 3, 128>; };

__device__ inline f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// SiLU(g) * u; the reciprocal is the hardware one (~1 ulp in fp32), far
// below the fp16 rounding of h that follows
__device__ inline float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Row of accumulator register r for lane `lane` in a 32x32 MFMA output tile.
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

struct Task {
  int e, row0, mcount, nt;
};

// Rows and format of expert e as every task lookup sees them. The caller's
// segment [offsets[e], offsets[e+1]) is clamped to [0, R) (bit
// MOE_FLAG_BAD_SEGMENT in *bad when that changes it), so no row outside the
// expert inputs, h or Y is ever addressed; an expert whose descriptor has
// another H or I than the call gets no rows (MOE_FLAG_EXPERT_SHAPE), so its
// packed matrices are never read with the call's sizes; an expert with rows
// whose format (or layout) no launch of the mask covers is reported
// (MOE_FLAG_FORMAT_NOT_LAUNCHED). Returns the format id of the expert's
// matrix in this role, or -1 when the role does not handle the expert (the
// fused gate/up role takes interleaved experts, the split roles the others).
template <int ROLE>
__device__ inline int expert_rows(const FfnArgs& a, int e, int& row0, int& count, uint32_t& bad) {
  // the descriptor's first 32 bytes: gate and down format words, H, I; up's
  // format word, the layout, the outlier counts
  const u32x4 d0 = reinterpret_cast<const u32x4*>(a.experts + e)[0];
  const u32x4 d1 = reinterpret_cast<const u32x4*>(a.experts + e)[1];
  const int o0 = a.offsets[e], o1 = a.offsets[e + 1];
  const int lo = min(max(o0, 0), a.R);
  const int hi = min(max(o1, lo), a.R);
  if (lo != o0 || hi != o1) bad |= MOE_FLAG_BAD_SEGMENT;
  int c = hi - lo;
  const bool split = d1[1] & MOE_PACK_SPLIT_GU;
  const uint32_t w = ROLE == R_DN ? d0[1] : (ROLE == R_UP ? d1[0] : d0[0]);
  const bool mine = ROLE == R_DN || (ROLE == R_GU ? !split : split);
  const int f = fmt_id(w & 0xff, (w >> 8) & 0xff, w >> 16);
  const bool gu = ROLE != R_DN;
  if (c > 0 && (d0[2] != (uint32_t)(gu ? a.K : a.N) || d0[3] != (uint32_t)(gu ? a.N : a.K))) {
    bad |= MOE_FLAG_EXPERT_SHAPE;
    c = 0;
  }
  if (c > 0) {
    if (mine && (f < 0 || !((a.fmt_mask >> f) & 1u))) bad |= MOE_FLAG_FORMAT_NOT_LAUNCHED;
    if (ROLE == R_GU && split && !(a.fmt_mask & kMaskSplitGU)) bad |= MOE_FLAG_FORMAT_NOT_LAUNCHED;
  }
  row0 = lo;
  count = c;
  return mine ? f : -1;
}

// The launch's matrix of expert ex, and its outlier list (rowptr, entries;
// false when it has none). Outlier list rows: gate/up rows 0..N-1 gate,
// N..2N-1 up; down rows 0..N-1.
template <int ROLE>
__device__ inline void role_matrix(const moe_packed_expert* ex, const uint8_t*& codes,
                                   const uint8_t*& params) {
  if constexpr (ROLE == R_DN) {
    codes = (const uint8_t*)ex->dn_codes;
    params = (const uint8_t*)ex->dn_params;
  } else if constexpr (ROLE == R_UP) {
    codes = (const uint8_t*)ex->up_codes;
    params = (const uint8_t*)ex->up_params;
  } else {
    codes = (const uint8_t*)ex->gu_codes;
    params = (const uint8_t*)ex->gu_params;
  }
}
template <int ROLE>
__device__ inline bool role_outliers(const moe_packed_expert* ex, const uint32_t*& rp,
                                     const OutEntry*& en) {
  const uint32_t n = __builtin_amdgcn_readfirstlane(ROLE == R_DN ? ex->n_out_dn : ex->n_out_gu);
  rp = (const uint32_t*)(ROLE == R_DN ? ex->out_dn_rowptr : ex->out_gu_rowptr);
  en = (const OutEntry*)(ROLE == R_DN ? ex->out_dn_entries : ex->out_gu_entries);
  return n > 0;
}
// outlier list row of a wavefront's output column (tile t of its pair, lane n)
template <int ROLE>
__device__ inline int outlier_row(int N, int unit, int t, int n) {
  if constexpr (ROLE == R_GU) return (t ? N : 0) + 32 * unit + n;
  else return (ROLE == R_UP ? N : 0) + 64 * unit + 32 * t + n;
}
// Task lookup over the experts of format `fid` (decode): tasks of expert e
// = ceil(count_e / BM) * NB, expert-major, then n-tile, then m-tile.
// The first block also flags experts with rows whose format is not in the
// launch mask (their rows would otherwise be left uncomputed).
template <int ROLE>
__device__ bool find_task(const FfnArgs& a, int fid, int BM, int NB, int L, Task& task) {
  __shared__ int s_wsum[16];  // up to 1024 threads
  __shared__ int s_res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_res[0] = -1;
  int cnt[2], ntk[2], r0[2];
  int local = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    int c = 0, f = -1, lo = 0;
    if (e < a.E) f = expert_rows<ROLE>(a, e, lo, c, bad);
    cnt[q] = c;
    r0[q] = lo;
    ntk[q] = f == fid ? ((c + BM - 1) / BM) * NB : 0;
    local += ntk[q];
  }
  if (bad && blockIdx.x == 0 && blockIdx.y == 0 && a.flags) atomicOr(a.flags, bad);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int start = incl - local;
  for (int w = 0; w < wave; ++w) start += s_wsum[w];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (L >= start && L < start + ntk[q]) {
      const int e = 2 * tid + q;
      const int rel = L - start;
      const int mt = (cnt[q] + BM - 1) / BM;
      const int mi = rel % mt;
      s_res[0] = e;
      s_res[1] = r0[q] + mi * BM;
      s_res[2] = min(BM, cnt[q] - mi * BM);
      s_res[3] = rel / mt;
    }
    start += ntk[q];
  }
  __syncthreads();
  // block-uniform: held in scalar registers, so what derives from them
  // (weight addresses, buffer descriptors) is computed on the scalar unit
  task.e = __builtin_amdgcn_readfirstlane(s_res[0]);
  task.row0 = __builtin_amdgcn_readfirstlane(s_res[1]);
  task.mcount = __builtin_amdgcn_readfirstlane(s_res[2]);
  task.nt = __builtin_amdgcn_readfirstlane(s_res[3]);
  return task.e >= 0;
}

// Task lookup of the prefill kernel for block b. Tasks are full m-tiles
// (count_e / BM per expert and n-tile) and partial last m-tiles (one per
// expert and n-tile when count_e is not a multiple of BM). Blocks are dealt
// round-robin to the 8 XCDs, and XCD x runs, in slot order, an equal
// contiguous share of the tasks that exist (not of the grid, which is an
// upper bound), in one of two orders:
//  - expert-major (a.lpt == 0): expert, then n-tile, then m-tile, so the
//    m-tiles sharing a weight tile run together and find it in L2;
//  - longest first (a.lpt == 1): a share of all full m-tiles, then a share
//    of the partial ones, so short blocks fill the tail of a launch that has
//    few blocks per slot.
// The grid needs 16 blocks more than there are tasks (spare blocks find
// nothing and exit).
template <int ROLE>
__device__ bool find_task_lpt(const FfnArgs& a, int fid, int BM, int NB, int b, Task& task) {
  __shared__ int s_wsum[2][16];  // up to 1024 threads
  __shared__ int s_res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  if (tid == 0) s_res[0] = -1;
  int cnt[2], nfu[2], npa[2], r0[2];
  int lf = 0, lp = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    int c = 0, f = -1, lo = 0;
    if (e < a.E) f = expert_rows<ROLE>(a, e, lo, c, bad);
    cnt[q] = c;
    r0[q] = lo;
    nfu[q] = f == fid ? (c / BM) * NB : 0;
    npa[q] = f == fid && c % BM ? NB : 0;
    lf += nfu[q];
    lp += npa[q];
  }
  if (bad && blockIdx.x == 0 && a.flags) atomicOr(a.flags, bad);
  int incf = lf, incp = lp;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int vf = __shfl_up(incf, off), vp = __shfl_up(incp, off);
    if (lane >= off) {
      incf += vf;
      incp += vp;
    }
  }
  if (lane == 63) {
    s_wsum[0][wave] = incf;
    s_wsum[1][wave] = incp;
  }
  __syncthreads();
  int sf = incf - lf, sp = incp - lp, F = 0, P = 0;
  for (int w = 0; w < nwaves; ++w) {
    if (w < wave) {
      sf += s_wsum[0][w];
      sp += s_wsum[1][w];
    }
    F += s_wsum[0][w];
    P += s_wsum[1][w];
  }
  const int x = b & 7, slot = b >> 3;
  if (!a.lpt) {
    // one list, expert-major; XCD x takes tasks [x q8 + min(x, r8), + n8)
    const int TOT = F + P;
    const int q8 = TOT >> 3, r8 = TOT & 7;
    const int n8 = q8 + (x < r8 ? 1 : 0);
    const int L = x * q8 + min(x, r8) + slot;
    if (slot < n8) {
      int st = sf + sp;  // the thread's experts start here in the combined list
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n = nfu[q] + npa[q];
        if (L >= st && L < st + n) {
          const int rel = L - st;
          const int mt = (cnt[q] + BM - 1) / BM;
          const int mi = rel % mt;
          s_res[0] = 2 * tid + q;
          s_res[1] = r0[q] + mi * BM;
          s_res[2] = min(BM, cnt[q] - mi * BM);
          s_res[3] = rel / mt;
        }
        st += n;
      }
    }
  } else {
    // the XCD's shares of the two lists
    const int qf = F >> 3, rf = F & 7, qp = P >> 3, rp = P & 7;
    const int nf = qf + (x < rf ? 1 : 0);
    const int bf = x * qf + min(x, rf);
    // the partial list's extras go to the last XCDs (the full list's to the
    // first), so no XCD takes two
    const int np = qp + (x >= 8 - rp ? 1 : 0);
    const int bp = x * qp + max(0, x - (8 - rp));
    const bool full = slot < nf;
    const int L = full ? bf + slot : bp + (slot - nf);
    if (full || slot - nf < np) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        const int st = full ? sf : sp;
        const int n = full ? nfu[q] : npa[q];
        if (L >= st && L < st + n) {
          const int rel = L - st;
          const int mf = cnt[q] / BM;  // full m-tiles of the expert
          const int mi = full ? rel % mf : mf;
          s_res[0] = e;
          s_res[1] = r0[q] + mi * BM;
          s_res[2] = min(BM, cnt[q] - mi * BM);
          s_res[3] = full ? rel / mf : rel;
        }
        sf += nfu[q];
        sp += npa[q];
      }
    }
  }
  __syncthreads();
  // block-uniform: held in scalar registers, so what derives from them
  // (weight addresses, buffer descriptors) is computed on the scalar unit
  task.e = __builtin_amdgcn_readfirstlane(s_res[0]);
  task.row0 = __builtin_amdgcn_readfirstlane(s_res[1]);
  task.mcount = __builtin_amdgcn_readfirstlane(s_res[2]);
  task.nt = __builtin_amdgcn_readfirstlane(s_res[3]);
  return task.e >= 0;
}

// Task lookup of the prefill kernel for a launch of less than two rounds of
// block slots: longest first in four classes. The tiles with 4 filled 32-row
// sub-tiles (full m-tiles, and partial ones of more than 3 BM / 4 rows) come
// first, then the partial tiles with 3, 2 and 1, so the shortest blocks make
// the tail. XCD x runs an equal contiguous share of each class in turn; a
// class's remainder goes to the XCDs after the previous class's, so no XCD
// takes more than one task above the others. (find_task_lpt holds the other
// orders; this one pays for four prefix sums instead of two.)
template <int ROLE>
__device__ bool find_task_lpt4(const FfnArgs& a, int fid, int BM, int NB, int b, Task& task) {
  constexpr int NC = 4;  // longest-first classes: 4, 3, 2, 1 filled sub-tiles
  __shared__ int s_wsum[NC][16];  // up to 1024 threads
  __shared__ int s_res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  if (tid == 0) s_res[0] = -1;
  const int SUB = BM / 4;  // rows of a sub-tile class step
  int cnt[2], ncl[2][NC], cls[2], r0[2];
  int lsum[NC] = {0, 0, 0, 0};
  uint32_t bad = 0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    int c = 0, f = -1, lo = 0;
    if (e < a.E) f = expert_rows<ROLE>(a, e, lo, c, bad);
    cnt[q] = c;
    r0[q] = lo;
    const bool mine = f == fid;
    const int rem = c % BM;
    // class of the partial tile: 0 (as long as a full one) .. 3 (shortest)
    cls[q] = rem ? NC - (rem + SUB - 1) / SUB : 0;
#pragma unroll
    for (int k = 0; k < NC; ++k) ncl[q][k] = 0;
    if (mine) {
      ncl[q][0] = (c / BM) * NB;
      if (rem) ncl[q][cls[q]] += NB;
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) lsum[k] += ncl[q][k];
  }
  if (bad && blockIdx.x == 0 && a.flags) atomicOr(a.flags, bad);
  int inc[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) inc[k] = lsum[k];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int v = __shfl_up(inc[k], off);
      if (lane >= off) inc[k] += v;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < NC; ++k) s_wsum[k][wave] = inc[k];
  }
  __syncthreads();
  int st[NC], tot[NC];  // the thread's experts' first task in each list; list sizes
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    st[k] = inc[k] - lsum[k];
    tot[k] = 0;
  }
  for (int w = 0; w < nwaves; ++w) {
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (w < wave) st[k] += s_wsum[k][w];
      tot[k] += s_wsum[k][w];
    }
  }
  const int x = b & 7, slot = b >> 3;
  {
    // XCD x's share of list k: q + 1 tasks on the r XCDs starting at `rot`
    // (the XCD after the previous list's extras), q on the others
    int rot = 0, before = 0;
    int k_sel = -1, L = 0;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int q = tot[k] >> 3, r = tot[k] & 7;
      const int d = (x - rot + 8) & 7;  // x's position counted from rot
      const int n = q + (d < r ? 1 : 0);
      // extras of the XCDs below x: those at positions < r among x' < x
      int ex = 0;
      for (int y = 0; y < x; ++y) ex += ((y - rot + 8) & 7) < r ? 1 : 0;
      if (k_sel < 0 && slot - before < n) {
        k_sel = k;
        L = x * q + ex + (slot - before);
      }
      before += n;
      rot = (rot + r) & 7;
    }
    if (k_sel >= 0) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int e = 2 * tid + q;
        int s0 = 0, n = 0;
#pragma unroll
        for (int k = 0; k < NC; ++k) {
          if (k == k_sel) {
            s0 = st[k];
            n = ncl[q][k];
          }
        }
        if (L >= s0 && L < s0 + n) {
          const int rel = L - s0;
          const int mf = cnt[q] / BM;  // full m-tiles of the expert
          int mi, nt;
          if (k_sel == 0) {
            // the expert's class-0 tiles: its full m-tiles, plus the partial
            // one when that is class 0 too
            const int mt = mf + ((cnt[q] % BM) && cls[q] == 0 ? 1 : 0);
            mi = rel % mt;
            nt = rel / mt;
          } else {
            mi = mf;
            nt = rel;
          }
          s_res[0] = e;
          s_res[1] = r0[q] + mi * BM;
          s_res[2] = min(BM, cnt[q] - mi * BM);
          s_res[3] = nt;
        }
        if (k_sel >= 0) {
#pragma unroll
          for (int k = 0; k < NC; ++k) st[k] += ncl[q][k];
        }
      }
    }
  }
  __syncthreads();
  // block-uniform: held in scalar registers, so what derives from them
  // (weight addresses, buffer descriptors) is computed on the scalar unit
  task.e = __builtin_amdgcn_readfirstlane(s_res[0]);
  task.row0 = __builtin_amdgcn_readfirstlane(s_res[1]);
  task.mcount = __builtin_amdgcn_readfirstlane(s_res[2]);
  task.nt = __builtin_amdgcn_readfirstlane(s_res[3]);
  return task.e >= 0;
}

// fp16 holds |v| <= 65504; beyond, the stored h is +-inf
constexpr float kF16Max = 65504.0f;

// stores h = silu(g) * u; true when h is stored as fp16 and overflows it
__device__ inline bool store_gu(const FfnArgs& a, int row, int col, float g, float u) {
  const float sc = a.ascale ? a.ascale[row] : 1.0f;
  const float h = silu_mul(g * sc, u * sc);
  if (a.out_f32) {
    reinterpret_cast<float*>(a.out)[(size_t)row * a.N + col] = h;
    return false;
  }
  reinterpret_cast<f16*>(a.out)[(size_t)row * a.N + col] = (f16)h;
  return fabsf(h) > kF16Max;
}

// split gate/up roles: the gate pass stores g (times the row's input scale)
// in h's buffer, the up pass replaces it with silu(g) * u; true when an fp16
// h overflows
template <int ROLE>
__device__ inline bool store_split(const FfnArgs& a, int row, int col, float v) {
  const float sc = a.ascale ? a.ascale[row] : 1.0f;
  const size_t i = (size_t)row * a.N + col;
  float h;
  if constexpr (ROLE == R_GATE) {
    h = v * sc;
  } else {
    const float g = a.out_f32 ? reinterpret_cast<const float*>(a.out)[i]
                              : (float)reinterpret_cast<const f16*>(a.out)[i];
    h = silu_mul(g, v * sc);
  }
  if (a.out_f32) {
    reinterpret_cast<float*>(a.out)[i] = h;
    return false;
  }
  reinterpret_cast<f16*>(a.out)[i] = (f16)h;
  return fabsf(h) > kF16Max;
}

__device__ inline void store_dn(const FfnArgs& a, int split, int row, int col, float y) {
  const float sc = a.ascale ? a.ascale[row] : 1.0f;
  reinterpret_cast<float*>(a.out)[((size_t)split * a.R + row) * a.N + col] = y * sc;
}

template <class F>
struct BTile {
  typename F::CodeT w0, w1;
  PBuf<F::EB> q0, q1;
};

// 16 bytes per lane from r at voff + soff into LDS at lds + 16 lane
__device__ inline void dma16(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// ===========================================================================
// Decode family
// ===========================================================================
// decode: outlier entries per batch (three keep the 4-bit kernels at three
// wavefronts per SIMD)
#ifndef MOEQ_DEC_OUTB
#define MOEQ_DEC_OUTB 3
#endif

// End of a decode wavefront: outlier corrections and stores of its two
// output tiles, for the accumulator registers r whose bit is set in `regs`
// (v0, v1: the tiles' register values, K partial sums already added).
template <class F, int ROLE>
__device__ inline void decode_finish(const FfnArgs& a, const Task& t, const moe_packed_expert* ex,
                                     rsrc_t rA, int rg, int split, int lane, uint32_t regs,
                                     float (&v0)[16], float (&v1)[16]) {
  const int n = lane & 31;
  bool over = false;
  // Outliers of the matrix, added once (by the K split that starts at 0):
  // per output column, each listed weight's correction times the rows'
  // inputs at its column. Entries go four at a time: their loads, then all
  // the rows' input loads of the four, then the products, so a list costs
  // a quarter as many memory round trips as its length.
  const uint32_t* orp;
  const OutEntry* oen;
  if (role_outliers<ROLE>(ex, orp, oen) && split == 0) {
    constexpr int B = MOEQ_DEC_OUTB;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int lr = outlier_row<ROLE>(a.N, rg, tt, n);
      const int b0 = (int)orp[lr], c = (int)orp[lr + 1] - b0;
      const OutEntry* en = oen + b0;
      for (int j = 0; j < c; j += B) {
        uint32_t kk[B];
        float dd[B];
#pragma unroll
        for (int u = 0; u < B; ++u) {
          const int e = min(j + u, c - 1);
          kk[u] = en[e].k;
          dd[u] = en[e].delta;
        }
        f16 x[B][16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!((regs >> r) & 1)) continue;
          const uint32_t ro = (uint32_t)(t.row0 + min(acc_row(r, lane), t.mcount - 1)) * a.K;
#pragma unroll
          for (int u = 0; u < B; ++u)
            x[u][r] = __builtin_bit_cast(f16, bload<uint16_t>(rA, (ro + kk[u]) * 2, 0));
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (j + u >= c) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (!((regs >> r) & 1)) continue;
            if (tt) v1[r] = fmaf(dd[u], (float)x[u][r], v1[r]);
            else v0[r] = fmaf(dd[u], (float)x[u][r], v0[r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (!((regs >> r) & 1)) continue;
    const int i = acc_row(r, lane);
    if (i < t.mcount) {
      const int row = t.row0 + i;
      if constexpr (ROLE == R_GU) {
        over |= store_gu(a, row, 32 * rg + n, v0[r], v1[r]);
      } else if constexpr (ROLE == R_DN) {
        store_dn(a, split, row, 64 * rg + n, v0[r]);
        store_dn(a, split, row, 64 * rg + 32 + n, v1[r]);
      } else {
        over |= store_split<ROLE>(a, row, 64 * rg + n, v0[r]);
        over |= store_split<ROLE>(a, row, 64 * rg + 32 + n, v1[r]);
      }
    }
  }
  if (over && a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_FP16_RANGE);
}

template <class F, int ROLE>
__global__ __launch_bounds__(kThreads) void ffn_decode_kernel(FfnArgs a, int ksw) {
  constexpr bool GU = ROLE == R_GU;
  // The 4 wavefronts of a block form 4/ksw row groups of ksw wavefronts; the
  // ksw wavefronts of a group split the K tiles of the block's K range and
  // meet in LDS. A row group is the gate/up pair (output tile j: row tiles
  // 2j, 2j+1) or the down row-tile pair (2j, 2j+1).
  __shared__ float red[4 * 2 * 16 * 64];
  const int G = 4 / ksw;
  const int NRG = GU ? a.N / 32 : a.N / 64;
  const int NB = (NRG + G - 1) / G;
  Task t;
  if (!find_task<ROLE>(a, F::ID, 32, NB, blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kh = lane >> 5;
  const int grp = wave / ksw, ks = wave % ksw;
  const int rg = t.nt * G + grp;
  const bool on = rg < NRG;
  const int KTn = a.K / F::KT;
  const int NE = a.K / F::GE;
  const moe_packed_expert* ex = a.experts + t.e;
  const uint8_t *codes, *params;
  role_matrix<ROLE>(ex, codes, params);
  const int rt0 = 2 * min(rg, NRG - 1);  // a group past the end streams a valid pair
  // 32-row weight tiles of the matrix (2I rows of interleaved gate/up, or H)
  const int NRT = GU ? 2 * a.N / 32 : a.N / 32;
  const rsrc_t rC = make_rsrc(uniform_ptr(codes), (uint32_t)((size_t)NRT * KTn * F::TB));
  const rsrc_t rP = make_rsrc(uniform_ptr(params), (uint32_t)((size_t)NRT * NE * 32 * F::EB));
  const uint32_t vc0 = (uint32_t)rt0 * KTn * F::TB + lane * F::CB;
  const uint32_t vc1 = vc0 + (uint32_t)KTn * F::TB;
  // 3-bit tiles: the lane's bytes of the high-bit plane
  const uint32_t vh0 = (uint32_t)rt0 * KTn * F::TB + F::HOFF + lane * 8;
  const uint32_t vh1 = vh0 + (uint32_t)KTn * F::TB;
  // group of the lane's first element in tile kt: kt KT / GE, plus kh SPAN / GE
  // when groups are no longer than a tile
  const uint32_t vp0 =
      ((uint32_t)rt0 * NE * 32 + n + (F::GE <= F::KT ? kh * (F::SPAN / F::GE) : 0) * 32) * F::EB;
  const uint32_t vp1 = vp0 + (uint32_t)NE * 32 * F::EB;

  const DeqConsts dk = make_deq_consts<F>();
  const int split = blockIdx.y;
  const int per = (KTn + a.splits - 1) / a.splits;
  const int kb = split * per, ke = min(KTn, kb + per);

  // Lanes of rows past the segment take an offset past the buffer's range:
  // their loads return zeros without a memory access (buffer range check),
  // and their MFMA rows are never stored. Those loads used to re-read the
  // tile's first row: at a few rows per expert most of the token-row loads,
  // which moved twice the weight bytes through each CU's load path.
  const bool arow = n < t.mcount;
  const rsrc_t rA = make_rsrc(a.a, (uint32_t)((size_t)a.R * a.K * 2));
  const uint32_t va = arow ? ((uint32_t)(t.row0 + n) * a.K + kh * F::SPAN) * 2 : kPastRange;

  struct AFrag {
    f16x8 v[F::STEPS];
  };
  // tiles of this wavefront: kt_i = kb + ks + ksw i, i < nt. Prefetches past
  // the last tile re-read a valid tile (result unused) so that the loop body
  // has no conditional loads and exact wait counts.
  const int nt = ke > kb + ks ? (ke - kb - ks + ksw - 1) / ksw : 0;
  auto tile_of = [&](int i) { return min(kb + ks + ksw * i, KTn - 1); };
  auto load_b = [&](int i, BTile<F>& b) {
    const int kt = tile_of(i);
    b.w0 = load_codes<F, kNT>(rC, vc0, vh0, (uint32_t)kt * F::TB);
    b.w1 = load_codes<F, kNT>(rC, vc1, vh1, (uint32_t)kt * F::TB);
    const uint32_t sp = (uint32_t)(kt * F::KT / F::GE) * 32 * F::EB;
    b.q0.template load<kNT>(rP, vp0, sp);
    b.q1.template load<kNT>(rP, vp1, sp);
  };
  auto load_a = [&](int i, AFrag& af) {
    const int kt = tile_of(i);
    // every lane loads: rows past the segment read zeros (offset past the
    // range), and their outputs (MFMA rows of their own) are never stored
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s)
      af.v[s] = bload<f16x8>(rA, va, (uint32_t)(kt * F::KT + 8 * s) * 2);
  };
  f32x16 acc0 = {}, acc1 = {};
  auto compute = [&](const BTile<F>& b, const AFrag& af) {
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
      const f16x8 b0 = dequant_step<F>(b.w0, b.q0, s, dk);
      const f16x8 b1 = dequant_step<F>(b.w1, b.q1, s, dk);
      acc0 = mfma32(af.v[s], b0, acc0);
      acc1 = mfma32(af.v[s], b1, acc1);
    }
  };
  // weights and token fragments two tiles ahead (three slots each)
  BTile<F> B0, B1, B2;
  AFrag A0, A1, A2;
  load_b(0, B0);
  load_a(0, A0);
  load_b(1, B1);
  load_a(1, A1);
  for (int i = 0; i < nt; i += 3) {
    load_b(i + 2, B2); load_a(i + 2, A2); compute(B0, A0);
    load_b(i + 3, B0); load_a(i + 3, A0); if (i + 1 < nt) compute(B1, A1);
    load_b(i + 4, B1); load_a(i + 4, A1); if (i + 2 < nt) compute(B2, A2);
  }

  // reduce the ksw partial sums of each row group: red[w][m][r][lane];
  // wavefront ks of a group finalises registers r = (16/ksw) ks .. +16/ksw.
  // Register r holds token rows 8(r/4) + (r%4) and that + 4 of the tile:
  // registers whose rows all lie past the segment are neither reduced nor
  // stored (at one token per expert only register 0 carries a row).
  const int mrows = __builtin_amdgcn_readfirstlane(t.mcount);
  auto live = [&](int r) { return 8 * (r >> 2) + (r & 3) < mrows; };
  if (ksw > 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (!live(r)) continue;
      red[((wave * 2 + 0) * 16 + r) * 64 + lane] = acc0[r];
      red[((wave * 2 + 1) * 16 + r) * 64 + lane] = acc1[r];
    }
    __syncthreads();
  }
  if (!on) return;
  const int RPW = 16 / ksw;
  const int w0 = grp * ksw;
  // this wavefront's rows: registers r of its K-split share that hold rows
  auto mine = [&](int r) { return r / RPW == ks && live(r); };
  float v0[16], v1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    v0[r] = acc0[r];
    v1[r] = acc1[r];
    if (!mine(r) || ksw == 1) continue;
    v0[r] = 0.f;
    v1[r] = 0.f;
    for (int w = 0; w < ksw; ++w) {
      v0[r] += red[(((w0 + w) * 2 + 0) * 16 + r) * 64 + lane];
      v1[r] += red[(((w0 + w) * 2 + 1) * 16 + r) * 64 + lane];
    }
  }
  uint32_t regs = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) regs |= mine(r) ? 1u << r : 0u;
  decode_finish<F, ROLE>(a, t, ex, rA, rg, split, lane, regs, v0, v1);
}

// Decode GEMV with a shared token tile (launches with short K streams or
// enough row groups to fill the device): the 4 wavefronts of a block own 4
// consecutive row groups and stream the same K tile of their weights at the
// same time, so the block's 32 token rows of that K tile reach LDS once, by
// DMA (buffer loads with an LDS destination), instead of once per wavefront
// through the vector memory path. The token-row loads of the per-wavefront
// kernel move twice the weight bytes through each CU's load path, from L2.
// LDS holds a ring of three token tiles: at the start of tile i a wavefront
// waits for its own DMA of tile i, the block meets at one barrier (every
// DMA of tile i has landed, every wavefront is done with tile i-1), then the
// DMA of tile i+2 goes into tile i-1's buffer and the weight codes of tile
// i+2 into tile i-1's register slot, and tile i is computed. Token rows are
// stored with their 16-byte chunks swizzled as in the prefill kernel, so the
// A-fragment reads of 16 lanes fall on 16 different 4-bank groups. The
// down projection's blocks take the K range of their split (blockIdx.y).
template <class F, int ROLE>
__global__ __launch_bounds__(kThreads) void ffn_decode_sa_kernel(FfnArgs a) {
  constexpr bool GU = ROLE == R_GU;
  constexpr int ROWB = F::KT * 2;              // bytes of a token row's K tile
  constexpr int TILEB = 32 * ROWB;             // 4 KiB (KT 64) or 8 KiB (KT 128)
  constexpr int CPR = F::KT / 8;               // 16-byte chunks per row
  constexpr int NI = TILEB / (kThreads * 16);  // DMA instructions per wavefront and tile
  constexpr int RPI = 64 / CPR;                // token rows one DMA instruction fills
  // three arrays, not one: the compiler can then tell that the DMA into one
  // buffer does not feed the reads of another and waits only where needed
  __shared__ __attribute__((aligned(1024))) uint8_t tk0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t tk1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t tk2[TILEB];
  const int NRG = GU ? a.N / 32 : a.N / 64;
  const int NB = (NRG + 3) / 4;
  Task t;
  if (!find_task<ROLE>(a, F::ID, 32, NB, blockIdx.x, t)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kh = lane >> 5;
  const int rg = t.nt * 4 + wave;
  const bool on = rg < NRG;
  const int KTn = a.K / F::KT;
  const int NE = a.K / F::GE;
  const moe_packed_expert* ex = a.experts + t.e;
  const uint8_t *codes, *params;
  role_matrix<ROLE>(ex, codes, params);
  const int rt0 = 2 * min(rg, NRG - 1);  // a group past the end streams a valid pair
  const int NRT = GU ? 2 * a.N / 32 : a.N / 32;
  const rsrc_t rC = make_rsrc(uniform_ptr(codes), (uint32_t)((size_t)NRT * KTn * F::TB));
  const rsrc_t rP = make_rsrc(uniform_ptr(params), (uint32_t)((size_t)NRT * NE * 32 * F::EB));
  const uint32_t vc0 = (uint32_t)rt0 * KTn * F::TB + lane * F::CB;
  const uint32_t vc1 = vc0 + (uint32_t)KTn * F::TB;
  const uint32_t vh0 = (uint32_t)rt0 * KTn * F::TB + F::HOFF + lane * 8;
  const uint32_t vh1 = vh0 + (uint32_t)KTn * F::TB;
  const uint32_t vp0 =
      ((uint32_t)rt0 * NE * 32 + n + (F::GE <= F::KT ? kh * (F::SPAN / F::GE) : 0) * 32) * F::EB;
  const uint32_t vp1 = vp0 + (uint32_t)NE * 32 * F::EB;
  const DeqConsts dk = make_deq_consts<F>();
  const rsrc_t rA = make_rsrc(a.a, (uint32_t)((size_t)a.R * a.K * 2));

  // DMA slots: instruction j of wavefront w fills slots [(w NI + j) 64, +64)
  // of a buffer, one 16-byte slot per lane; slot -> (row, stored chunk) ->
  // logical chunk. Rows past the segment take an offset past the buffer's
  // range (no memory access; their LDS rows feed MFMA rows that are never
  // stored). A wavefront whose slots hold only such rows issues no DMA at
  // all (block-uniform per wavefront, so its wait counts stay exact).
  auto swz = [](int r) { return CPR == 8 ? (r >> 1) & 7 : r & 15; };
  const bool dma_on = wave * NI * RPI < t.mcount;
  uint32_t doff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int slot = (wave * NI + j) * 64 + lane;
    const int r = slot / CPR, pc = slot % CPR;
    const int c = pc ^ swz(r);
    doff[j] = r < t.mcount ? (uint32_t)(((size_t)(t.row0 + r) * a.K + 8 * c) * 2) : kPastRange;
  }
  const int split = blockIdx.y;
  const int per = (KTn + a.splits - 1) / a.splits;
  const int kb = split * per, nt = max(min(KTn, kb + per) - kb, 0);
  auto tile_of = [&](int i) { return min(kb + i, KTn - 1); };
  auto load_b = [&](int i, BTile<F>& b) {
    const int kt = tile_of(i);
    b.w0 = load_codes<F, kNT>(rC, vc0, vh0, (uint32_t)kt * F::TB);
    b.w1 = load_codes<F, kNT>(rC, vc1, vh1, (uint32_t)kt * F::TB);
    const uint32_t sp = (uint32_t)(kt * F::KT / F::GE) * 32 * F::EB;
    b.q0.template load<kNT>(rP, vp0, sp);
    b.q1.template load<kNT>(rP, vp1, sp);
  };
  f32x16 acc0 = {}, acc1 = {};
  auto compute = [&](const uint8_t* buf, const BTile<F>& b) {
    f16x8 av[F::STEPS];
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
      const int c = (kh * (F::SPAN / 8) + s) ^ swz(n);
      av[s] = *reinterpret_cast<const f16x8*>(buf + n * ROWB + c * 16);
    }
#pragma unroll
    for (int s = 0; s < F::STEPS; ++s) {
      const f16x8 b0 = dequant_step<F>(b.w0, b.q0, s, dk);
      const f16x8 b1 = dequant_step<F>(b.w1, b.q1, s, dk);
      acc0 = mfma32(av[s], b0, acc0);
      acc1 = mfma32(av[s], b1, acc1);
    }
  };
  // memory operations per tile: this wavefront's DMA instructions (if it
  // has any), then the weight loads (codes and parameters of two row tiles)
  constexpr int LPT = 2 * code_loads<F>() + 2;
  // The loop is instantiated with and without the DMA, so that the compiler's
  // own wait counts (for the weight registers) are exact on each path: with
  // one loop whose DMA is conditional, it waits on both paths as if the DMA
  // were missing, i.e. for the last DMA and more weight loads than needed.
  auto run = [&](auto dma_c) {
    constexpr bool D = decltype(dma_c)::value;
    auto dma = [&](int i, uint8_t* buf) {
      if constexpr (D) {
        const uint32_t so = (uint32_t)tile_of(i) * ROWB;
#pragma unroll
        for (int j = 0; j < NI; ++j) dma16(rA, buf + (wave * NI + j) * 1024, doff[j], so);
      }
    };
    // in flight at the start of tile i: weights i, DMA i+1, weights i+1
    constexpr int VM = 2 * LPT + (D ? NI : 0);
    auto step = [&](int i, const uint8_t* cur, uint8_t* nxt2, const BTile<F>& cb, BTile<F>& nb2) {
      if constexpr (D) __builtin_amdgcn_s_waitcnt(0x0F70 | (VM & 15) | ((VM >> 4) << 14));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      dma(i + 2, nxt2);
      load_b(i + 2, nb2);
      compute(cur, cb);
    };
    // the nt tiles of the split's K range; prefetches past its end re-read
    // a valid tile (unused)
    BTile<F> B0, B1, B2;
    dma(0, tk0);
    load_b(0, B0);
    dma(1, tk1);
    load_b(1, B1);
    // whole rounds of three tiles, then the last one or two: no branch
    // inside the loop body, so its wait counts are the steady state's
    int i = 0;
    for (; i + 3 <= nt; i += 3) {
      step(i, tk0, tk2, B0, B2);
      step(i + 1, tk1, tk0, B1, B0);
      step(i + 2, tk2, tk1, B2, B1);
    }
    if (i < nt) step(i, tk0, tk2, B0, B2);
    if (i + 1 < nt) step(i + 1, tk1, tk0, B1, B0);
    // no DMA may still be in flight when the block's LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);
  };
  if (dma_on)
    run(IntC<1>{});
  else
    run(IntC<0>{});
  if (!on) return;
  const int mrows = __builtin_amdgcn_readfirstlane(t.mcount);
  uint32_t regs = 0;
  float v0[16], v1[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    v0[r] = acc0[r];
    v1[r] = acc1[r];
    regs |= 8 * (r >> 2) + (r & 3) < mrows ? 1u << r : 0u;
  }
  decode_finish<F, ROLE>(a, t, ex, rA, rg, split, lane, regs, v0, v1);
}

// decode: fewest K tiles a wavefront of a K-split group streams
#ifndef MOEQ_DEC_MINT
#define MOEQ_DEC_MINT 16
#endif
// decode: rounds of block slots the shared-token-tile kernel's gate/up
// blocks must fill (fewer: Mixtral-shaped gate/up at 8 tokens, 1.02 rounds,
// measured 5% slower on it, at 32 tokens, 1.17 rounds, 5% faster)
#ifndef MOEQ_DEC_SA_ROUNDS
#define MOEQ_DEC_SA_ROUNDS 2
#endif
// decode: longest per-wavefront stream (K tiles) for which the
// shared-token-tile kernel runs from one round of block slots
#ifndef MOEQ_DEC_SA_SHORT
#define MOEQ_DEC_SA_SHORT 32
#endif


// ===========================================================================
// Prefill family
// ===========================================================================
// Prefill tuning knobs (defaults measured best on MI355X): the three-buffer
// pipeline for 16 KiB token tiles, wavefronts per block. Weight loads are
// cached: the m-tiles of an expert re-read each weight tile.
#ifndef MOEQ_PF_DEEP
#define MOEQ_PF_DEEP 1
#endif
#ifndef MOEQ_PF_WAVES
#define MOEQ_PF_WAVES 4
#endif
// MOEQ_PF_BM: token rows per block (256 puts one wavefront on each SIMD and
// measured ~20% slower; 64 spills at four blocks per CU)
#ifndef MOEQ_PF_BM
#define MOEQ_PF_BM 128
#endif
constexpr int kBM = MOEQ_PF_BM;
constexpr int kMT = kBM / 32;  // 32-row sub-tiles per block tile
// wavefronts per prefill block: they share one token tile in LDS, each
// streaming its own 64 weight rows (one block per CU at 8)
constexpr int kPW = MOEQ_PF_WAVES;
constexpr int kBPC = (8 / kPW) * 128 / kBM;  // blocks per CU
// bytes of LDS a prefill wavefront stages its output through: 16 rows of 64
// fp32 at a pitch of 72
constexpr int kStageB = 16 * 72 * 4;

// LPT4: the four-class longest-first lookup (down launches of less than two
// rounds); a separate instantiation, so the other launches keep the kernel
// that the lighter lookup compiles to
template <class F, int ROLE, bool LPT4 = false>
__global__ __launch_bounds__(64 * kPW, kBPC) void ffn_prefill_kernel(FfnArgs a) {
  constexpr bool GU = ROLE == R_GU;
  // Token tile in LDS: kBM rows x KT halves, rows packed (KT*2 bytes) with the
  // 16-byte chunks of row r stored at chunk ^ swz(r). The LDS serves a 16-byte
  // read of 16 lanes (16 consecutive rows, one logical chunk) per cycle from
  // 64 banks; swz makes those 16 reads land on 16 different 4-bank groups.
  constexpr int ROWB = F::KT * 2;
  constexpr int TILEB = kBM * ROWB;           // 16 KiB (4-bit) or 32 KiB (2-bit)
  constexpr int CPR = F::KT / 8;              // 16-byte chunks per row
  constexpr int NI = TILEB / (kPW * 64 * 16);  // LDS-DMA instructions per wave and tile
  // two separate arrays: the compiler can then tell that a DMA into one
  // buffer does not feed reads of the other, and waits only where needed
  // 16 KiB tiles (4-bit) get three buffers and a deeper pipeline
  constexpr bool DEEP = MOEQ_PF_DEEP && 3 * TILEB * kBPC <= 160 * 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[DEEP ? TILEB : 16];
  // unit of one wavefront: gate/up output tile j (row tiles 2j, 2j+1), or
  // the down row-tile pair (2j, 2j+1); a block covers kPW consecutive units
  const int NU = a.N / (GU ? 32 : 64);
  const int NB = (NU + kPW - 1) / kPW;
  Task t;
  bool found;
  if constexpr (LPT4)
    found = find_task_lpt4<ROLE>(a, F::ID, kBM, NB, blockIdx.x, t);
  else
    found = find_task_lpt<ROLE>(a, F::ID, kBM, NB, blockIdx.x, t);
  if (!found) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kh = lane >> 5;
  const int KTn = a.K / F::KT;
  const int NE = a.K / F::GE;
  const moe_packed_expert* ex = a.experts + t.e;
  const uint8_t *codes, *params;
  role_matrix<ROLE>(ex, codes, params);
  const int unit = kPW * t.nt + wave;
  const bool on = unit < NU;
  // a wavefront past the last unit streams a valid tile and discards it, so
  // every wavefront runs the same straight-line loop
  const int rt0 = 2 * unit;
  const int rtl = 2 * min(unit, NU - 1);
  // 32-row weight tiles of the matrix (2I rows of interleaved gate/up, or H);
  // the descriptors span the whole matrix
  const int NRT = GU ? 2 * a.N / 32 : a.N / 32;
  const rsrc_t rC = make_rsrc(uniform_ptr(codes), (uint32_t)((size_t)NRT * KTn * F::TB));
  const rsrc_t rP = make_rsrc(uniform_ptr(params), (uint32_t)((size_t)NRT * NE * 32 * F::EB));
  const rsrc_t rA = make_rsrc(a.a, (uint32_t)((size_t)a.R * a.K * 2));
  const uint32_t vc0 = (uint32_t)rtl * KTn * F::TB + lane * F::CB;
  const uint32_t vc1 = vc0 + (uint32_t)KTn * F::TB;
  // 3-bit tiles: the lane's bytes of the high-bit plane
  const uint32_t vh0 = (uint32_t)rtl * KTn * F::TB + F::HOFF + lane * 8;
  const uint32_t vh1 = vh0 + (uint32_t)KTn * F::TB;
  // the group of a lane's first element in tile kt is kt KT / GE plus, when
  // groups are no longer than a tile, its half's kh SPAN / GE
  const uint32_t vp0 =
      ((uint32_t)rtl * NE * 32 + n + (F::GE <= F::KT ? kh * (F::SPAN / F::GE) : 0) * 32) * F::EB;
  const uint32_t vp1 = vp0 + (uint32_t)NE * 32 * F::EB;

  const DeqConsts dk = make_deq_consts<F>();
  // Token tile DMA: the block's instruction g fills LDS slots [64 g, +64) of
  // the buffer, one 16-byte slot per lane. Slot -> (row, stored chunk) ->
  // logical chunk; rows past the segment repeat its last row (their outputs
  // are never stored). Offsets are in bytes from the start of K tile kt of
  // the token matrix. The NQ instructions of each 32-row sub-tile per
  // wavefront are shared out over the wavefronts (instruction j of
  // wavefront w: sub-tile j / NQ, g = (j / NQ) NQ kPW + (j % NQ) kPW + w),
  // so a partial m-tile with AMT filled sub-tiles loads only those, with
  // the same AMT NQ instructions on every wavefront (exact wait counts).
  // 128-byte rows: two rows per 64 banks, so rows 2i and 2i+1 share a chunk
  // pattern and differ in bank half; 256-byte rows fill all banks each.
  static_assert(NI % kMT == 0 && (NI / kMT) * kPW * 64 == 32 * CPR, "DMA instructions per sub-tile");
  constexpr int NQ = NI / kMT;
  auto swz = [](int r) { return CPR == 8 ? (r >> 1) & 7 : r & 15; };
  auto dslot = [&](int j) { return (j / NQ) * NQ * kPW + (j % NQ) * kPW + wave; };
  uint32_t doff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int slot = dslot(j) * 64 + lane;
    const int r = slot / CPR, pc = slot % CPR;
    const int c = pc ^ swz(r);
    doff[j] = (uint32_t)(((size_t)(t.row0 + min(r, t.mcount - 1)) * a.K + 8 * c) * 2);
  }
  // the DMA of K tile kt's first AMT sub-tiles
  auto dma_a = [&](int kt, uint8_t* buf, auto amt_c) {
#pragma unroll
    for (int j = 0; j < decltype(amt_c)::value * NQ; ++j)
      dma16(rA, buf + dslot(j) * 1024, doff[j], (uint32_t)kt * ROWB);
  };
  auto load_b = [&](int kt, BTile<F>& b) {
    b.w0 = load_codes<F>(rC, vc0, vh0, (uint32_t)kt * F::TB);
    b.w1 = load_codes<F>(rC, vc1, vh1, (uint32_t)kt * F::TB);
    const uint32_t sp = (uint32_t)(kt * F::KT / F::GE) * 32 * F::EB;
    b.q0.load(rP, vp0, sp);
    b.q1.load(rP, vp1, sp);
  };
  // The block's pipeline, specialised on the number of 32-row sub-tiles
  // that hold rows (the last m-tile of an expert is usually partial): empty
  // sub-tiles cost no MFMAs and no LDS reads. amt is block-uniform, taken
  // through a scalar register so every wavefront branches the same way.
  const int amt = __builtin_amdgcn_readfirstlane((t.mcount + 31) / 32);
  auto run = [&](auto amt_c) {
    constexpr int AMT = decltype(amt_c)::value;
    f32x16 acc[AMT][2];
#pragma unroll
    for (int mi = 0; mi < AMT; ++mi) {
      acc[mi][0] = f32x16{};
      acc[mi][1] = f32x16{};
    }
    // Outliers of the matrix, before the K loop (the accumulators start from
    // the corrections, while few other registers are live): each listed
    // weight's correction (delta = its fp16 value - the decoded weight)
    // times the token rows' inputs at its column. The inputs come from the transposed copy, where the block's
    // rows of one column are contiguous and in accumulator order: lane
    // (n, kh) reads its 16 rows of sub-tile mi as 32 bytes, so one entry
    // costs 2 AMT 16-byte loads that touch two cache lines per lane pair
    // (row-major inputs cost one line per row). Each output column's list
    // is walked with the next entry loaded while the current one's inputs
    // are in flight. Rows past the segment read the last row's inputs, as
    // the token tile does.
    {
      const uint32_t* orp;
      const OutEntry* oen;
      if (on && role_outliers<ROLE>(ex, orp, oen)) {
        if (!a.at) {
          if (tid == 0 && a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_FORMAT_NOT_LAUNCHED);
        } else {
          const int lo = min(max(a.offsets[t.e], 0), a.R);
          const rsrc_t rT = make_rsrc(a.at, (uint32_t)((size_t)a.K * a.rp * 2));
          const uint32_t pb = (uint32_t)(a.poff[t.e] + (t.row0 - lo) + 16 * kh) * 2;
          const uint32_t rowT = (uint32_t)a.rp * 2;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int lr = outlier_row<ROLE>(a.N, unit, tt, n);
            const int b0 = (int)orp[lr], c = (int)orp[lr + 1] - b0;
            // the entries' columns and deltas as separate scalars, so they
            // stay in registers
            const OutEntry* en = oen + b0;
            uint32_t qk = c > 0 ? en[0].k : 0u;
            float qd = c > 0 ? en[0].delta : 0.f;
            for (int j = 0; j < c; ++j) {
              f16x8 v[AMT][2];
#pragma unroll
              for (int mi = 0; mi < AMT; ++mi) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
                  v[mi][hf] = bload<f16x8>(rT, qk * rowT + pb, (uint32_t)(32 * mi + 8 * hf) * 2);
              }
              const bool more = j + 1 < c;
              const uint32_t nk = more ? en[j + 1].k : qk;
              const float nd = more ? en[j + 1].delta : qd;
#pragma unroll
              for (int mi = 0; mi < AMT; ++mi) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                  acc[mi][tt][r] = fmaf(qd, (float)v[mi][r >> 3][r & 7], acc[mi][tt][r]);
              }
              qk = nk;
              qd = nd;
            }
          }
        }
      }
    }
    // fragment (mi, step s) of lane (n, kh): row mi*32 + n, logical chunk
    // kh*SPAN/8 + s; swz(mi*32 + n) == swz(n)
    auto afrag = [&](const uint8_t* buf, int mi, int s) {
      const int c = (kh * (F::SPAN / 8) + s) ^ swz(n);
      return *reinterpret_cast<const f16x8*>(buf + (mi * 32 + n) * ROWB + c * 16);
    };

    // Pipeline, one barrier per K tile. At the start of tile kt the wavefront
    // waits for its own DMA of token tile kt and its weight codes of tile kt
    // (everything but the 4 weight loads of tile kt+1 issued at the end of
    // tile kt-1), then the barrier makes every wavefront's DMA visible and
    // frees the other buffer; the DMA of tile kt+1 goes out, tile kt is
    // computed (codes of MFMA step s+1 decoded while the MFMAs of step s run),
    // and the weight codes of tile kt+2 are fetched into the slot just used.
    // Prefetches past the last tile re-read the last tile (unused).
    BTile<F> R0, R1;  // raw weight codes (tile parity)
    auto mma_jit = [&](const uint8_t* buf, const BTile<F>& raw) {
      f16x8 av[AMT];
#pragma unroll
      for (int mi = 0; mi < AMT; ++mi) av[mi] = afrag(buf, mi, 0);
      f16x8 d0 = dequant_step<F>(raw.w0, raw.q0, 0, dk);
      f16x8 d1 = dequant_step<F>(raw.w1, raw.q1, 0, dk);
#pragma unroll
      for (int s = 0; s < F::STEPS; ++s) {
        f16x8 an[AMT];
        f16x8 n0 = d0, n1 = d1;
        if (s + 1 < F::STEPS) {
#pragma unroll
          for (int mi = 0; mi < AMT; ++mi) an[mi] = afrag(buf, mi, s + 1);
          n0 = dequant_step<F>(raw.w0, raw.q0, s + 1, dk);
          n1 = dequant_step<F>(raw.w1, raw.q1, s + 1, dk);
        }
        // (a wavefront with no row tile of its own computes on the clamped
        // tile and stores nothing: no branch around the matrix-core chain)
#pragma unroll
        for (int mi = 0; mi < AMT; ++mi) {
          acc[mi][0] = mfma32(av[mi], d0, acc[mi][0]);
          acc[mi][1] = mfma32(av[mi], d1, acc[mi][1]);
        }
        if (s + 1 < F::STEPS) {
#pragma unroll
          for (int mi = 0; mi < AMT; ++mi) av[mi] = an[mi];
        }
        d0 = n0;
        d1 = n1;
        // one scheduling region per step: each MFMA of step s is followed by
        // a share of step s+1's decode, so a lone wavefront keeps the matrix
        // core fed while it decodes (about 2/3 of the decode is pinned behind
        // the MFMAs; the scheduler places the rest and the LDS reads, which
        // measured 1-4% faster than pinning all of them)
        constexpr int NM = 2 * AMT;
        constexpr int VPM = (24 + NM - 1) / NM;
        constexpr int VG = VPM > 2 ? VPM - 1 : VPM;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VG, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (DEEP) {
      // Three token buffers, three weight slots: the DMA of token tile kt+2
      // goes out at the start of tile kt (into the buffer tile kt-1 used) and
      // the weight codes of tile kt+3 at its end, so both are fetched two full
      // tiles ahead. At the start of tile kt everything but the last
      // 2 LPT + AMT NQ memory operations (weights kt+1, DMA kt+1, weights
      // kt+2) has landed.
      BTile<F> R2;
      // memory operations of one tile's weights (codes of two row tiles and
      // their parameters); weights kt+1, DMA kt+1 and weights kt+2 may stay
      // in flight
      constexpr int LPT = 2 * code_loads<F>() + 2;
      constexpr int VM = 2 * LPT + AMT * NQ;
      auto tile = [&](int kt, uint8_t* cur, uint8_t* next2, BTile<F>& slot) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | (VM & 15) | ((VM >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma_a(min(kt + 2, KTn - 1), next2, amt_c);
        mma_jit(cur, slot);
        load_b(min(kt + 3, KTn - 1), slot);
      };
      load_b(0, R0);
      dma_a(0, lds0, amt_c);
      load_b(min(1, KTn - 1), R1);
      dma_a(min(1, KTn - 1), lds1, amt_c);
      load_b(min(2, KTn - 1), R2);
      int kt = 0;
      for (; kt + 2 < KTn; kt += 3) {
        tile(kt, lds0, lds2, R0);
        tile(kt + 1, lds1, lds0, R1);
        tile(kt + 2, lds2, lds1, R2);
      }
      if (kt < KTn) tile(kt, lds0, lds2, R0);
      if (kt + 1 < KTn) tile(kt + 1, lds1, lds0, R1);
    } else {
      // Two token buffers: the DMA of token tile kt+1 goes out at the start of
      // tile kt, the weight codes of tile kt+2 at its end.
      auto tile_start = [&](int kt, uint8_t* next) {
        // vmcnt(LPT): the weight loads of tile kt+1 may stay in flight
        constexpr int LPT = 2 * code_loads<F>() + 2;
        __builtin_amdgcn_s_waitcnt(0x0F70 | LPT);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // past the last tile this re-fills the idle buffer (no branch in the loop)
        dma_a(min(kt + 1, KTn - 1), next, amt_c);
      };
      dma_a(0, lds0, amt_c);
      load_b(0, R0);
      load_b(min(1, KTn - 1), R1);
      int kt = 0;
      for (; kt + 1 < KTn; kt += 2) {
        tile_start(kt, lds1);
        mma_jit(lds0, R0);
        load_b(min(kt + 2, KTn - 1), R0);
        tile_start(kt + 1, lds0);
        mma_jit(lds1, R1);
        load_b(min(kt + 3, KTn - 1), R1);
      }
      if (kt < KTn) {
        tile_start(kt, lds1);
        mma_jit(lds0, R0);
      }
    }
    // no LDS DMA may still be in flight when the block's LDS is released
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Epilogue, staged through LDS 16 rows at a time so each lane stores 16
    // bytes of a row instead of one element: a wavefront's output rows are 64
    // fp32 (down) or 32 fp16/fp32 (gate/up) values held one column per lane,
    // and one-element stores made the end of a block slow (20% of the
    // short-K down launches). Each wavefront writes its own 4.5 KiB of the
    // token buffers (wavefronts 0/1 in lds0, 2/3 in lds1) once every
    // wavefront is past its last token tile. Row pitches are padded so rows
    // r and r+4, written by the two lane halves, fall on different banks.
    static_assert(kPW <= 4 && 2 * kStageB <= TILEB, "epilogue staging exceeds the token buffers");
    __syncthreads();
    if (!on) return;
    uint8_t* stg = (wave >> 1 ? lds1 : lds0) + (wave & 1) * kStageB;
    bool over = false;  // an fp16 h out of range (rows past the segment
                        // repeat its last row, so they add no false report)
#pragma unroll
    for (int mi = 0; mi < AMT; ++mi) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int i0 = mi * 32 + 16 * hh;  // first tile row of this half
        // a wavefront's LDS operations run in order: the fences only keep
        // the compiler from moving reads of other lanes' values across writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
        for (int r = 8 * hh; r < 8 * hh + 8; ++r) {
          const int lr = 8 * ((r >> 2) & 1) + 4 * kh + (r & 3);  // == acc_row(r) - 16 hh
          if constexpr (GU) {
            const float sc = (a.ascale && i0 + lr < t.mcount) ? a.ascale[t.row0 + i0 + lr] : 1.0f;
            const float h = silu_mul(acc[mi][0][r] * sc, acc[mi][1][r] * sc);
            if (a.out_f32) {
              reinterpret_cast<float*>(stg)[lr * 36 + n] = h;
            } else {
              reinterpret_cast<f16*>(stg)[lr * 40 + n] = (f16)h;
              over |= fabsf(h) > kF16Max;
            }
          } else {
            reinterpret_cast<float*>(stg)[lr * 72 + n] = acc[mi][0][r];
            reinterpret_cast<float*>(stg)[lr * 72 + 32 + n] = acc[mi][1][r];
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (GU) {
          if (a.out_f32) {
            // 16 rows x 32 fp32: 8 lanes per row, two stores
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int lr = 8 * j + (lane >> 3), c4 = lane & 7;
              const float4 v = *reinterpret_cast<const float4*>(stg + (lr * 36 + 4 * c4) * 4);
              if (i0 + lr < t.mcount)
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) +
                                           (size_t)(t.row0 + i0 + lr) * a.N + 32 * unit + 4 * c4) = v;
            }
          } else {
            // 16 rows x 32 fp16: 4 lanes per row, one store
            const int lr = lane >> 2, c8 = lane & 3;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + (lr * 40 + 8 * c8) * 2);
            if (i0 + lr < t.mcount)
              *reinterpret_cast<uint4*>(reinterpret_cast<f16*>(a.out) +
                                        (size_t)(t.row0 + i0 + lr) * a.N + 32 * unit + 8 * c8) = v;
          }
        } else {
          // 16 rows x 64 fp32: 16 lanes per row, four stores
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int lr = 4 * j + (lane >> 4), c4 = lane & 15;
            float4 v = *reinterpret_cast<const float4*>(stg + (lr * 72 + 4 * c4) * 4);
            if (i0 + lr < t.mcount) {
              const float sc = a.ascale ? a.ascale[t.row0 + i0 + lr] : 1.0f;
              v.x *= sc;
              v.y *= sc;
              v.z *= sc;
              v.w *= sc;
              const size_t o = (size_t)(t.row0 + i0 + lr) * a.N + 32 * rt0 + 4 * c4;
              if constexpr (ROLE == R_DN) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o) = v;
              } else {
                // split gate/up: g into h's buffer, or h = silu(g) * u in place
                if constexpr (ROLE == R_UP) {
                  float4 g;
                  if (a.out_f32) {
                    g = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.out) + o);
                  } else {
                    const f16x4 g16 = *reinterpret_cast<const f16x4*>(reinterpret_cast<const f16*>(a.out) + o);
                    g = float4{(float)g16[0], (float)g16[1], (float)g16[2], (float)g16[3]};
                  }
                  v.x = silu_mul(g.x, v.x);
                  v.y = silu_mul(g.y, v.y);
                  v.z = silu_mul(g.z, v.z);
                  v.w = silu_mul(g.w, v.w);
                }
                if (a.out_f32) {
                  *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o) = v;
                } else {
                  *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(a.out) + o) =
                      f16x4{(f16)v.x, (f16)v.y, (f16)v.z, (f16)v.w};
                  over |= fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))) > kF16Max;
                }
              }
            }
          }
        }
      }
    }
    if (ROLE != R_DN && over && a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_FP16_RANGE);
  };
  if (amt > 3 * kMT / 4)
    run(IntC<kMT>{});
  else if (amt > kMT / 2)
    run(IntC<(3 * kMT / 4 > 1 ? 3 * kMT / 4 : 1)>{});
  else if (amt > kMT / 4)
    run(IntC<(kMT / 2 > 1 ? kMT / 2 : 1)>{});
  else
    run(IntC<(kMT / 4 > 1 ? kMT / 4 : 1)>{});
}

inline int max_tiles(int R, int E, int BM) { return (R + BM - 1) / BM + (R < E ? R : E); }

// compute units of the current device
inline int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

template <int FID, int ROLE>
hipError_t launch_one(const FfnArgs& a, bool decode, hipStream_t s) {
  using F = typename FmtOf<FID>::T;
  constexpr bool GU = ROLE == R_GU;
  constexpr bool DN = ROLE == R_DN;
  if (decode) {
    // The shared-token-tile kernel, whose blocks (one per touched expert,
    // set of 4 row groups and K split, counting each touched expert as one
    // 32-row tile) stream every K tile of their split on each wavefront:
    //  * when those streams are short (at most MOEQ_DEC_SA_SHORT K tiles)
    //    and the blocks fill at least one round of the device's block slots:
    //    the 256-expert layers at 64 tokens (down 15-21%, gate/up 6-16%
    //    faster), where the per-wavefront kernel splits K little or not at
    //    all and so has about as many blocks;
    //  * for gate/up, when the blocks fill at least MOEQ_DEC_SA_ROUNDS
    //    rounds (W4A8 at 16 tokens: 4% faster). With fewer rounds the long
    //    blocks leave a slow tail (Mixtral gate/up at 8 tokens, 1.02 rounds:
    //    7% slower); its down launches, long streams over few blocks, were
    //    slower on it at every size measured;
    //  * for any launch when the caller's mask asks for it.
    {
      const int NRG = GU ? a.N / 32 : a.N / 64;
      const int KTw = (a.K / F::KT + a.splits - 1) / a.splits;
      const long sa_blocks = (long)(a.R < a.E ? a.R : a.E) * ((NRG + 3) / 4) * a.splits;
      int bpc = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, (const void*)ffn_decode_sa_kernel<F, ROLE>,
                                                       kThreads, 0) != hipSuccess || bpc <= 0)
        bpc = 1;
      const long slots = (long)device_cus() * bpc;
      if ((a.fmt_mask & kMaskSharedTile) || (KTw <= MOEQ_DEC_SA_SHORT && sa_blocks >= slots) ||
          (!DN && sa_blocks >= MOEQ_DEC_SA_ROUNDS * slots)) {
        dim3 grid(max_tiles(a.R, a.E, 32) * ((NRG + 3) / 4), DN ? a.splits : 1);
        hipLaunchKernelGGL((ffn_decode_sa_kernel<F, ROLE>), grid, dim3(kThreads), 0, s, a);
        return hipGetLastError();
      }
    }
    // wavefronts splitting K inside a block: as many as keep >= 16 K tiles
    // (per split) on each; when few weight rows are in flight (a handful of
    // tokens on small experts) streams of >= 8 tiles on more wavefronts
    const int KTn = a.K / F::KT / (DN ? a.splits : 1);
    const int NRG = GU ? a.N / 32 : a.N / 64;
    int ksw = KTn >= 4 * MOEQ_DEC_MINT ? 4 : (KTn >= 2 * MOEQ_DEC_MINT ? 2 : 1);
    const long groups = (long)(a.R < a.E ? a.R : a.E) * NRG * (DN ? a.splits : 1);
    while (ksw < 4 && groups * ksw < 2048 && KTn >= 2 * ksw * (MOEQ_DEC_MINT / 2)) ksw *= 2;
    // blocks (one per touched expert and row-group set, as when each touched
    // expert has at most 32 rows) that would spill a little past one round
    // of the device's block slots: half as many, on twice longer K streams,
    // so the launch ends after one round (one token: 1.5 us of 37)
    if (ksw > 1) {
      const long blocks = groups / (4 / ksw);
      int bpc = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, (const void*)ffn_decode_kernel<F, ROLE>,
                                                       kThreads, 0) != hipSuccess || bpc <= 0)
        bpc = 1;
      const long slots = (long)device_cus() * bpc;
      if (blocks > slots && blocks <= 2 * slots) ksw /= 2;
    }
    const int NB = (NRG + 4 / ksw - 1) / (4 / ksw);
    dim3 grid(max_tiles(a.R, a.E, 32) * NB, DN ? a.splits : 1);
    hipLaunchKernelGGL((ffn_decode_kernel<F, ROLE>), grid, dim3(kThreads), 0, s, a, ksw);
  } else {
    const int NU = a.N / (GU ? 32 : 64);
    const int NB = (NU + kPW - 1) / kPW;
    // longest-first order when the launch has fewer than 4 blocks per block
    // slot of the device (its tail is then a large share of its time); for
    // the down projection in four classes below 2 blocks per slot
    const long nblk = (long)max_tiles(a.R, a.E, kBM) * NB;
    FfnArgs b = a;
    const long slots = (long)device_cus() * kBPC;
    b.lpt = nblk < 2 * slots ? 2 : (nblk < 4 * slots ? 1 : 0);
    // 16 spare blocks: the per-XCD task shares may round up (find_task_lpt)
    dim3 grid(nblk + 16);
    if constexpr (DN) {
      if (b.lpt == 2) {
        hipLaunchKernelGGL((ffn_prefill_kernel<F, R_DN, true>), grid, dim3(64 * kPW), 0, s, b);
        return hipGetLastError();
      }
    }
    if (b.lpt == 2) b.lpt = 1;  // the two-class order
    hipLaunchKernelGGL((ffn_prefill_kernel<F, ROLE, false>), grid, dim3(64 * kPW), 0, s, b);
  }
  return hipGetLastError();
}

// every role of format FID
template <int FID>
hipError_t launch_roles(int role, const FfnArgs& a, bool decode, hipStream_t s) {
  switch (role) {
    case R_GU: return launch_one<FID, R_GU>(a, decode, s);
    case R_DN: return launch_one<FID, R_DN>(a, decode, s);
    case R_GATE: return launch_one<FID, R_GATE>(a, decode, s);
    case R_UP: return launch_one<FID, R_UP>(a, decode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace moeq
