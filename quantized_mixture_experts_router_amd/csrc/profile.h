// Routing profile and precision tiers (profile.hip).
#pragma once

#include "common.h"

namespace moeq {

// per-expert counts of ids[0..n) in [0, E), added into hist[E] (device)
hipError_t launch_expert_histogram(const int32_t* ids, long n, int E, int64_t* hist,
                                   hipStream_t s);
// host only; false when every expert at the last tier exceeds the budget
bool plan_tiers(const int64_t* counts, int E, const uint64_t* tier_bytes, int ntiers,
                uint64_t budget, int32_t* tier_of, uint64_t* used_out);

}  // namespace moeq
