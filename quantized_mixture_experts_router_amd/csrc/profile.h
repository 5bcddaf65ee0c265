// Routing profile and precision tiers (profile.hip); int8 router logits
// and their calibration range (route.hip).
#pragma once

#include "common.h"

namespace moeq {

// per-expert counts of ids[0..n) in [0, E), added into hist[E] (device)
hipError_t launch_expert_histogram(const int32_t* ids, long n, int E, int64_t* hist,
                                   hipStream_t s);
// host only; false when every expert at the last tier exceeds the budget
bool plan_tiers(const int64_t* counts, int E, const uint64_t* tier_bytes, int ntiers,
                uint64_t budget, int32_t* tier_of, uint64_t* used_out);

// int8 router logits: top-k over the affine int8 round trip of the logits
// (partials P as launch_route_logits leaves them), and the calibration range
hipError_t launch_route_topk_q(const double* P, int KB, const float* b, int T, int E, int k,
                               const float* qscale, const int32_t* qzero, int32_t* ids, float* w,
                               float* logits, hipStream_t s);
hipError_t launch_logit_range(const double* P, int KB, const float* b, int T, int E, double* lo,
                              double* hi, hipStream_t s);

}  // namespace moeq
