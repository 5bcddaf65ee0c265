// Grouped expert GEMMs of the e2m1 block formats (groups 16, 32, 64, 128).
#include "fused_impl.h"

namespace moeq {

hipError_t launch_ffn_e4(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s) {
  switch (fid) {
    case F_E4G16: return launch_roles<F_E4G16>(role, a, decode, s);
    case F_E4G32: return launch_roles<F_E4G32>(role, a, decode, s);
    case F_E4G64: return launch_roles<F_E4G64>(role, a, decode, s);
    case F_E4G128: return launch_roles<F_E4G128>(role, a, decode, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused_e4(int fid, const FusedArgs& fa, hipStream_t s) {
  switch (fid) {
    case F_E4G16: return launch_fused_one<F_E4G16>(fa, s);
    case F_E4G32: return launch_fused_one<F_E4G32>(fa, s);
    case F_E4G64: return launch_fused_one<F_E4G64>(fa, s);
    case F_E4G128: return launch_fused_one<F_E4G128>(fa, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moeq
