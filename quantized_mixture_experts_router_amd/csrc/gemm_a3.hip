// Grouped expert GEMMs of the asymmetric 3-bit block formats (groups 16, 32, 64, 128).
#include "fused_impl.h"

namespace moeq {

hipError_t launch_ffn_a3(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s) {
  switch (fid) {
    case F_A3G16: return launch_roles<F_A3G16>(role, a, decode, s);
    case F_A3G32: return launch_roles<F_A3G32>(role, a, decode, s);
    case F_A3G64: return launch_roles<F_A3G64>(role, a, decode, s);
    case F_A3G128: return launch_roles<F_A3G128>(role, a, decode, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused_a3(int fid, const FusedArgs& fa, hipStream_t s) {
  switch (fid) {
    case F_A3G16: return launch_fused_one<F_A3G16>(fa, s);
    case F_A3G32: return launch_fused_one<F_A3G32>(fa, s);
    case F_A3G64: return launch_fused_one<F_A3G64>(fa, s);
    case F_A3G128: return launch_fused_one<F_A3G128>(fa, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moeq
