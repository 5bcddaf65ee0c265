// Dispatch of the grouped expert GEMMs: one launch per block format present
// in the call's mask and per role (fused gate/up + SwiGLU for experts whose
// gate and up share a format; split gate then up for the others; down).
// The kernels live in gemm_impl.h, instantiated per format family.
#include "common.h"
#include "fused_impl.h"

namespace moeq {

hipError_t launch_ffn_a4(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a2(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_e4(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a1(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a3(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);

hipError_t launch_fused_a4(int fid, const FusedArgs& fa, hipStream_t s);
hipError_t launch_fused_a2(int fid, const FusedArgs& fa, hipStream_t s);
hipError_t launch_fused_e4(int fid, const FusedArgs& fa, hipStream_t s);
hipError_t launch_fused_a1(int fid, const FusedArgs& fa, hipStream_t s);
hipError_t launch_fused_a3(int fid, const FusedArgs& fa, hipStream_t s);

hipError_t launch_ffn_i8(int fid, int role, const FfnArgs& a, hipStream_t s);

hipError_t launch_ffn_fmt(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s) {
  switch (fid / 4) {
    case 0: return launch_ffn_a4(fid, role, a, decode, s);
    case 1: return launch_ffn_a2(fid, role, a, decode, s);
    case 2: return launch_ffn_e4(fid, role, a, decode, s);
    case 3: return launch_ffn_a1(fid, role, a, decode, s);
    case 4: return launch_ffn_a3(fid, role, a, decode, s);
  }
  return hipErrorInvalidValue;
}

namespace {

// one launch per format of the mask; with int8 operands, the int8 kernels
// take the W4A8 formats of the fused gate/up and down roles at prefill
hipError_t launch_all(int role, const FfnArgs& a, bool decode, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  for (int f = 0; f < F_COUNT; ++f) {
    if ((a.fmt_mask >> f) & 1u) {
      const bool i8 = !decode && a.a8 && ((kI8Formats >> f) & 1u) && (role == R_GU || role == R_DN);
      const hipError_t e = i8 ? launch_ffn_i8(f, role, a, s) : launch_ffn_fmt(f, role, a, decode, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_ffn_gate_up(const moe_packed_expert* experts, const int32_t* offsets,
                              uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E,
                              int k, const f16* a16, const float* ascale, void* h, int h_f32,
                              bool decode, const OutlierInputs& oi, const I8Inputs& i8,
                              hipStream_t s) {
  FfnArgs a;
  a.a8 = i8.a8;
  a.asum = i8.asum;
  a.at = oi.at;
  a.rp = oi.rp;
  a.poff = oi.poff;
  a.experts = experts;
  a.offsets = offsets;
  a.flags = flags;
  a.fmt_mask = fmt_mask;
  a.E = E;
  a.K = H;
  a.N = I;
  a.a = a16;
  a.ascale = ascale;
  a.out = h;
  a.out_f32 = h_f32;
  a.R = T * k;
  a.splits = 1;
  a.lpt = 0;
  hipError_t e = launch_all(R_GU, a, decode, s);
  if (e == hipSuccess && (fmt_mask & kMaskSplitGU)) {
    // experts with separate gate and up streams: g first, then h in place
    e = launch_all(R_GATE, a, decode, s);
    if (e == hipSuccess) e = launch_all(R_UP, a, decode, s);
  }
  return e;
}

// K tile and parameter entry widths of format id f (host)
static void fmt_tile(int f, int& kt, int& ge) {
  const int fam = f / 4, group = 16 << (f % 4);
  const int span = (fam == 0 || fam == 2) ? 32 : 64;  // 4-bit and e2m1 : 2-, 1-, 3-bit
  kt = 2 * span;
  ge = group > span ? group : span;
}

hipError_t launch_ffn_fused(const moe_packed_expert* experts, const int32_t* offsets,
                            uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                            const f16* a16, const float* ascale, float* yp, int S_plan,
                            int ns_plan, int* ns_used, hipStream_t s) {
  // the smallest admissible S >= the plan's for every format present
  int S = 0;
  for (int c = S_plan; c <= I && c <= 512 && !S; c = c == 64 ? 128 : c + 128) {
    if (I % c != 0) continue;
    bool ok = true;
    for (int f = 0; f < F_COUNT && ok; ++f) {
      if (!((fmt_mask >> f) & 1u)) continue;
      int kt, ge;
      fmt_tile(f, kt, ge);
      ok = c % kt == 0 && c % ge == 0;
    }
    if (ok) S = c;
  }
  if (!S || I / S > ns_plan) return hipErrorNotSupported;
  FusedArgs fa;
  FfnArgs& a = fa.g;
  a.experts = experts;
  a.offsets = offsets;
  a.flags = flags;
  a.fmt_mask = fmt_mask;
  a.E = E;
  a.K = H;
  a.N = I;
  a.a = a16;
  a.ascale = ascale;
  a.out = nullptr;
  a.out_f32 = 0;
  a.R = T * k;
  a.splits = 1;
  a.lpt = 0;
  fa.yp = yp;
  fa.S = S;
  fa.ns = I / S;
  *ns_used = fa.ns;
  for (int f = 0; f < F_COUNT; ++f) {
    if (!((fmt_mask >> f) & 1u)) continue;
    hipError_t e;
    switch (f / 4) {
      case 0: e = launch_fused_a4(f, fa, s); break;
      case 1: e = launch_fused_a2(f, fa, s); break;
      case 2: e = launch_fused_e4(f, fa, s); break;
      case 3: e = launch_fused_a1(f, fa, s); break;
      default: e = launch_fused_a3(f, fa, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_ffn_down(const moe_packed_expert* experts, const int32_t* offsets,
                           uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                           const f16* ain, const float* ascale, float* yp, int splits,
                           bool decode, const OutlierInputs& oi, const I8Inputs& i8,
                           hipStream_t s) {
  FfnArgs a;
  a.a8 = i8.a8;
  a.asum = i8.asum;
  a.at = oi.at;
  a.rp = oi.rp;
  a.poff = oi.poff;
  a.experts = experts;
  a.offsets = offsets;
  a.flags = flags;
  a.fmt_mask = fmt_mask;
  a.E = E;
  a.K = I;
  a.N = H;
  a.a = ain;
  a.ascale = ascale;
  a.out = yp;
  a.out_f32 = 1;
  a.R = T * k;
  a.splits = decode ? splits : 1;
  a.lpt = 0;
  return launch_all(R_DN, a, decode, s);
}

}  // namespace moeq
