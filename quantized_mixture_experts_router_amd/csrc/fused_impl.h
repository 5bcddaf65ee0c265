// Fused decode FFN: gate/up + SwiGLU + down of small batches in one launch.
//
// A block owns one touched expert (at most 32 rows: batches of up to 32
// tokens) and one slice of S columns of its intermediate dimension. Phase 1
// streams the expert's gate and up rows of that slice over all of K = H and
// leaves h = silu(g) * u of the slice, for every row of the expert, in LDS;
// phase 2 streams the down matrix's columns of the same slice (all H output
// rows, K = the slice) and writes the slice's share of Y into a partial sum
// plane of its own, yp[slice][row][H]. A reduction then adds the planes in a
// fixed order, with the top-k weights (combine_slices_kernel). Against a
// gate/up launch followed by a down launch, the down weights stream while
// other blocks still stream gate/up, with one block start and one task
// lookup instead of two; the cost is the partial planes (sized on the host
// to a few percent of the weight bytes). Scope table, first "next" row
// (single-launch decode; the mixed-precision notes, section 3.6, capture
// the layer in a graph and fuse the expert's linear with its activation).
#pragma once

#include "gemm_impl.h"

namespace moeq {

struct FusedArgs {
  FfnArgs g;  // gate/up view: K = H, N = I, a = expert inputs, ascale, flags
  float* yp;  // partial planes [ns][R][H]
  int S;      // slice width (columns of I)
  int ns;     // slices
};

namespace {

constexpr int kFusedRedBytes = 4 * 2 * 16 * 64 * 4;
// LDS bytes of a block for slice width S
inline size_t fused_lds_bytes(int S) {
  return (S < 128 ? kFusedRedBytes : 0) + (size_t)32 * (S + 8) * 2;
}

template <class F>
__global__ __launch_bounds__(kThreads, 2) void ffn_fused_decode_kernel(FusedArgs fa) {
  const FfnArgs& a = fa.g;
  const int H = a.K, I = a.N, S = fa.S;
  // LDS: the phase 1 K-split partials (32 KiB, only when S = 64 splits K),
  // then the h slice in fp16
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* red = reinterpret_cast<float*>(smem);
  const int hpitch = S + 8;  // halves per LDS row (padding spreads the rows over banks)
  f16* hs = reinterpret_cast<f16*>(smem + (S < 128 ? kFusedRedBytes : 0));

  Task t;
  if (!find_task<R_GU>(a, F::ID, 32, fa.ns, blockIdx.x, t)) return;
  const int j = t.nt;  // slice

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kh = lane >> 5;
  const moe_packed_expert* ex = a.experts + t.e;
  const DeqConsts dk = make_deq_consts<F>();
  const int mrows = __builtin_amdgcn_readfirstlane(t.mcount);
  auto live = [&](int r) { return 8 * (r >> 2) + (r & 3) < mrows; };
  const rsrc_t rA = make_rsrc(a.a, (uint32_t)((size_t)a.R * H * 2));
  struct AFrag {
    f16x8 v[F::STEPS];
  };
  bool over = false;

  // ---------------------------------------------------------------- phase 1
  {
    const int U = S / 32;                  // gate/up output tiles of the slice
    const int ksw = U >= 4 ? 1 : 4 / U;    // wavefronts splitting K per tile
    const int upw = U >= 4 ? U / 4 : 1;    // tiles per wavefront
    const int u0 = U >= 4 ? wave * upw : wave / ksw;
    const int ks = U >= 4 ? 0 : wave % ksw;
    const int KTn = H / F::KT, NE = H / F::GE;
    const int NRT = 2 * I / 32;
    const rsrc_t rC = make_rsrc(uniform_ptr(ex->gu_codes), (uint32_t)((size_t)NRT * KTn * F::TB));
    const rsrc_t rP =
        make_rsrc(uniform_ptr(ex->gu_params), (uint32_t)((size_t)NRT * NE * 32 * F::EB));
    // rows past the segment: an offset past the buffer's range (zeros, no
    // memory access; their MFMA rows are never stored)
    const uint32_t va = n < t.mcount ? ((uint32_t)(t.row0 + n) * H + kh * F::SPAN) * 2 : kPastRange;
    // tiles of this wavefront: unit u0 + i / per, K tile ks + ksw (i % per)
    const int per = (KTn - ks + ksw - 1) / ksw;
    const int nt = upw * per;
    auto unit_of = [&](int i) { return u0 + min(i, nt - 1) / per; };
    auto kt_of = [&](int i) { return ks + ksw * (min(i, nt - 1) % per); };
    auto load_b = [&](int i, BTile<F>& b) {
      const int gu = j * U + unit_of(i);  // global output tile: row tiles 2gu, 2gu + 1
      const int kt = kt_of(i);
      const uint32_t base = (uint32_t)(2 * gu) * KTn * F::TB;
      const uint32_t so = (uint32_t)kt * F::TB;
      b.w0 = load_codes<F, kNT>(rC, base + lane * F::CB, base + F::HOFF + lane * 8, so);
      b.w1 = load_codes<F, kNT>(rC, base + (uint32_t)KTn * F::TB + lane * F::CB,
                                base + (uint32_t)KTn * F::TB + F::HOFF + lane * 8, so);
      const uint32_t vp0 = ((uint32_t)(2 * gu) * NE * 32 + n +
                            (F::GE <= F::KT ? kh * (F::SPAN / F::GE) : 0) * 32) * F::EB;
      const uint32_t sp = (uint32_t)(kt * F::KT / F::GE) * 32 * F::EB;
      b.q0.template load<kNT>(rP, vp0, sp);
      b.q1.template load<kNT>(rP, vp0 + (uint32_t)NE * 32 * F::EB, sp);
    };
    auto load_a = [&](int i, AFrag& af) {
      const int kt = kt_of(i);
#pragma unroll
      for (int s = 0; s < F::STEPS; ++s)
        af.v[s] = bload<f16x8>(rA, va, (uint32_t)(kt * F::KT + 8 * s) * 2);
    };
    f32x16 acc0 = {}, acc1 = {};
    // one tile's MFMAs, then, after the last K tile of an output tile, its
    // SwiGLU into the LDS slice (K-split partials meet in LDS first)
    auto finish = [&](int u) {
      if (ksw > 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!live(r)) continue;
          red[((wave * 2 + 0) * 16 + r) * 64 + lane] = acc0[r];
          red[((wave * 2 + 1) * 16 + r) * 64 + lane] = acc1[r];
        }
        __syncthreads();
      }
      const int RPW = 16 / ksw, w0 = (wave / ksw) * ksw;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r / RPW != ks || !live(r)) continue;
        float g = acc0[r], v = acc1[r];
        if (ksw > 1) {
          g = 0.f;
          v = 0.f;
          for (int w = 0; w < ksw; ++w) {
            g += red[(((w0 + w) * 2 + 0) * 16 + r) * 64 + lane];
            v += red[(((w0 + w) * 2 + 1) * 16 + r) * 64 + lane];
          }
        }
        const int i = acc_row(r, lane);
        if (i < t.mcount) {
          const float sc = a.ascale ? a.ascale[t.row0 + i] : 1.0f;
          const float h = silu_mul(g * sc, v * sc);
          hs[i * hpitch + u * 32 + n] = (f16)h;
          over |= fabsf(h) > kF16Max;
        }
      }
      acc0 = f32x16{};
      acc1 = f32x16{};
    };
    auto compute = [&](int i, const BTile<F>& b, const AFrag& af) {
#pragma unroll
      for (int s = 0; s < F::STEPS; ++s) {
        const f16x8 b0 = dequant_step<F>(b.w0, b.q0, s, dk);
        const f16x8 b1 = dequant_step<F>(b.w1, b.q1, s, dk);
        acc0 = mfma32(af.v[s], b0, acc0);
        acc1 = mfma32(af.v[s], b1, acc1);
      }
      if (i % per == per - 1) finish(unit_of(i));
    };
    BTile<F> B0, B1, B2;
    AFrag A0, A1, A2;
    load_b(0, B0);
    load_a(0, A0);
    load_b(1, B1);
    load_a(1, A1);
    for (int i = 0; i < nt; i += 3) {
      load_b(i + 2, B2); load_a(i + 2, A2); compute(i, B0, A0);
      load_b(i + 3, B0); load_a(i + 3, A0); if (i + 1 < nt) compute(i + 1, B1, A1);
      load_b(i + 4, B1); load_a(i + 4, A1); if (i + 2 < nt) compute(i + 2, B2, A2);
    }
  }
  // ---------------------------------------------------------------- phase 2
  // (its first two weight tiles are requested before the barrier that
  // completes the h slice: they do not depend on it)
  {
    const int P = H / 64;              // output row-tile pairs of down
    const int KS = S / F::KT;          // K tiles of the slice
    const int kt0 = j * KS;
    const int KTn = I / F::KT, NE = I / F::GE;
    const int NRT = H / 32;
    const rsrc_t rC = make_rsrc(uniform_ptr(ex->dn_codes), (uint32_t)((size_t)NRT * KTn * F::TB));
    const rsrc_t rP =
        make_rsrc(uniform_ptr(ex->dn_params), (uint32_t)((size_t)NRT * NE * 32 * F::EB));
    const int npairs = (P - wave + 3) / 4;  // pairs wave, wave + 4, ...
    const int nt = npairs * KS;
    auto pair_of = [&](int i) { return wave + 4 * (min(i, nt - 1) / KS); };
    auto kt_of = [&](int i) { return kt0 + min(i, nt - 1) % KS; };
    auto load_b = [&](int i, BTile<F>& b) {
      const int p = pair_of(i), kt = kt_of(i);
      const uint32_t base = (uint32_t)(2 * p) * KTn * F::TB;
      const uint32_t so = (uint32_t)kt * F::TB;
      b.w0 = load_codes<F, kNT>(rC, base + lane * F::CB, base + F::HOFF + lane * 8, so);
      b.w1 = load_codes<F, kNT>(rC, base + (uint32_t)KTn * F::TB + lane * F::CB,
                                base + (uint32_t)KTn * F::TB + F::HOFF + lane * 8, so);
      const uint32_t vp0 = ((uint32_t)(2 * p) * NE * 32 + n +
                            (F::GE <= F::KT ? kh * (F::SPAN / F::GE) : 0) * 32) * F::EB;
      const uint32_t sp = (uint32_t)(kt * F::KT / F::GE) * 32 * F::EB;
      b.q0.template load<kNT>(rP, vp0, sp);
      b.q1.template load<kNT>(rP, vp0 + (uint32_t)NE * 32 * F::EB, sp);
    };
    f32x16 acc0 = {}, acc1 = {};
    float* yp = fa.yp + (size_t)j * a.R * H;
    auto compute = [&](int i, const BTile<F>& b) {
      const int kl = (i % KS) * F::KT;  // column of the K tile inside the slice
#pragma unroll
      for (int s = 0; s < F::STEPS; ++s) {
        const f16x8 av = *reinterpret_cast<const f16x8*>(hs + n * hpitch + kl + kh * F::SPAN + 8 * s);
        const f16x8 b0 = dequant_step<F>(b.w0, b.q0, s, dk);
        const f16x8 b1 = dequant_step<F>(b.w1, b.q1, s, dk);
        acc0 = mfma32(av, b0, acc0);
        acc1 = mfma32(av, b1, acc1);
      }
      if (i % KS == KS - 1) {
        const int p = pair_of(i);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!live(r)) continue;
          const int ii = acc_row(r, lane);
          if (ii < t.mcount) {
            float* yr = yp + (size_t)(t.row0 + ii) * H + 64 * p;
            yr[n] = acc0[r];
            yr[32 + n] = acc1[r];
          }
        }
        acc0 = f32x16{};
        acc1 = f32x16{};
      }
    };
    BTile<F> B0, B1, B2;
    load_b(0, B0);
    load_b(1, B1);
    __syncthreads();  // the h slice is complete
    for (int i = 0; i < nt; i += 3) {
      load_b(i + 2, B2); compute(i, B0);
      load_b(i + 3, B0); if (i + 1 < nt) compute(i + 1, B1);
      load_b(i + 4, B1); if (i + 2 < nt) compute(i + 2, B2);
    }
  }
  if (over && a.flags) atomicOr(a.flags, (uint32_t)MOE_FLAG_FP16_RANGE);
}

// Launch of format FID over the experts of that format (S, ns from the host;
// S a multiple of the format's K tile and parameter entry).
template <int FID>
hipError_t launch_fused_one(const FusedArgs& fa, hipStream_t s) {
  using F = typename FmtOf<FID>::T;
  // 64, or a multiple of 128 (the slice's output tiles divide among 4 waves)
  if (fa.S % F::KT != 0 || fa.S % F::GE != 0 || (fa.S != 64 && fa.S % 128 != 0) || fa.S > 512)
    return hipErrorNotSupported;
  // S = 64 splits each tile's K over two wavefronts, which meet at a barrier:
  // each must own at least one K tile
  if (fa.S < 128 && fa.g.K / F::KT < 2) return hipErrorNotSupported;
  const int rows = fa.g.R < fa.g.E ? fa.g.R : fa.g.E;  // touched experts, at most
  const size_t lds = fused_lds_bytes(fa.S);
  hipLaunchKernelGGL((ffn_fused_decode_kernel<F>), dim3(rows * fa.ns), dim3(kThreads), lds, s, fa);
  return hipGetLastError();
}

}  // namespace
}  // namespace moeq
