// The layer entry point that allocates nothing: moe_layer_forward with its
// workspace in a file-scope device array instead of a caller buffer, for
// callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends. Host code never uses the array's name as an address: the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// looked up once per device on the first call made with that device current,
// and only that address reaches kernels.
#include <mutex>

#include "common.h"

namespace moeq {
namespace {

__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  hipError_t status = hipErrorNotInitialized;
  void* ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// Address of the current device's copy of `scratch`, or nullptr.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.status == hipSuccess) d.ptr = p;
  });
  return d.status == hipSuccess ? d.ptr : nullptr;
}

}  // namespace
}  // namespace moeq

using namespace moeq;

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return MOE_NOALLOC_SCRATCH_BYTES; }

moe_status moe_layer_forward_noalloc(const void* x, moe_dtype xdt, const float* Wr, const float* b,
                                     const moe_packed_expert* experts, uint32_t fmt_mask, int T,
                                     int H, int I, int E, int k, moe_actq aq, void* out,
                                     moe_dtype out_dt, int32_t* topk_ids, float* topk_w,
                                     uint32_t* flags, void* stream) {
  WsLayout L;
  moe_status st = check_layer_sizes(T, H, I, E, k, aq, fmt_mask, L);
  if (st != MOE_OK) return st;
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (flags && ((uintptr_t)flags % 4) != 0) return MOE_ERR_ALIGNMENT;
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  return layer_forward_ws(x, xdt, Wr, b, experts, fmt_mask, T, H, I, E, k, aq, out, out_dt,
                          topk_ids, topk_w, ws, L, flags, (hipStream_t)stream);
}

}  // extern "C"
