// Dispatch of the grouped expert GEMMs: one launch per block format present
// in the call's mask and per role (fused gate/up + SwiGLU for experts whose
// gate and up share a format; split gate then up for the others; down).
// The kernels live in gemm_impl.h, instantiated per format family.
#include "common.h"
#include "gemm_impl.h"

namespace moeq {

hipError_t launch_ffn_a4(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a2(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_e4(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a1(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);
hipError_t launch_ffn_a3(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s);

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

// one launch per format of the mask
hipError_t launch_all(int role, const FfnArgs& a, bool decode, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  for (int f = 0; f < F_COUNT; ++f) {
    if ((a.fmt_mask >> f) & 1u) {
      const hipError_t e = launch_ffn_fmt(f, role, a, decode, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_ffn_gate_up(const moe_packed_expert* experts, const int32_t* offsets,
                              uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E,
                              int k, const f16* a16, const float* ascale, void* h, int h_f32,
                              bool decode, hipStream_t s) {
  FfnArgs a;
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

hipError_t launch_ffn_down(const moe_packed_expert* experts, const int32_t* offsets,
                           uint32_t fmt_mask, uint32_t* flags, int T, int H, int I, int E, int k,
                           const f16* ain, const float* ascale, float* yp, int splits,
                           bool decode, hipStream_t s) {
  FfnArgs a;
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
