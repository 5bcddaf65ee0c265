// The int8 prefill GEMMs (gemm_i8.h) of the two W4A8 formats.
#include "gemm_i8.h"

namespace moeq {

hipError_t launch_ffn_i8(int fid, int role, const FfnArgs& a, hipStream_t s) {
  if (fid == F_A4G128 && role == R_GU) return launch_i8_one<R_GU, 128>(a, s);
  if (fid == F_A4G128 && role == R_DN) return launch_i8_one<R_DN, 128>(a, s);
  return hipErrorNotSupported;
}

}  // namespace moeq
