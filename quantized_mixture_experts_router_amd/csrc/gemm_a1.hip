// Grouped expert GEMMs of the asymmetric 1-bit block formats (groups 16, 32, 64, 128).
#include "gemm_impl.h"

namespace moeq {

hipError_t launch_ffn_a1(int fid, int role, const FfnArgs& a, bool decode, hipStream_t s) {
  switch (fid) {
    case F_A1G16: return launch_roles<F_A1G16>(role, a, decode, s);
    case F_A1G32: return launch_roles<F_A1G32>(role, a, decode, s);
    case F_A1G64: return launch_roles<F_A1G64>(role, a, decode, s);
    case F_A1G128: return launch_roles<F_A1G128>(role, a, decode, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moeq
