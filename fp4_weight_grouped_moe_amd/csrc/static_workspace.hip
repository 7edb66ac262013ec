// moe_w4a16_fused_static_workspace: the fused layer for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// The workspace moe_w4a16_fused takes from its caller lives here instead, in one file-scope
// device array of MOE_STATIC_WORKSPACE_BYTES that every GPU the library runs on holds from
// the code object's load until the process ends. Its device address is looked up once per
// device with that device current (the array's name in host code is only a host-side stand-in,
// never a device address) and kept per device; the kernels get that pointer exactly as they
// get a caller's workspace. Nothing here allocates or frees memory. The fused kernels write
// every workspace region they read earlier in the same call (the FC2 arrival counts are
// zeroed by the FC1 launch, the work-queue counters by the route pack), so the array needs no
// clearing between calls. All calls on one GPU share its array: calls that overlap on one GPU
// (two streams, two threads) race and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe_w4a16.h"
#include "kernels.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];      // device address of `scratch` on each device, once looked up

}  // namespace

extern "C" int moe_w4a16_fused_static_workspace(const moe_w4a16_dims* dims, const void* prepared,
                                                size_t prepared_bytes, const uint16_t* x, int64_t m,
                                                const int32_t* topk_ids, const float* topk_weights, int topk,
                                                const int32_t* expert_map, int num_global_experts,
                                                int64_t token_capacity, uint16_t* out, hipStream_t stream) {
  size_t need = 0;
  if (int rc = moe_w4a16_workspace_size(dims, token_capacity, topk, &need); rc != MOE_OK) return rc;
  if (need > size_t(MOE_STATIC_WORKSPACE_BYTES))
    return moe::report_error(MOE_ERR_WORKSPACE,
                             "static workspace: this layer at token_capacity %lld needs %zu bytes, above the "
                             "library's %zu-byte device array (use moe_w4a16_fused with a caller workspace)",
                             (long long)token_capacity, need, size_t(MOE_STATIC_WORKSPACE_BYTES));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return moe::report_error(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return moe::report_error(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return moe::report_error(MOE_ERR_HIP, "hipGetSymbolAddress of the static workspace failed on device %d: %s",
                                 dev, hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return moe_w4a16_fused(dims, prepared, prepared_bytes, x, m, topk_ids, topk_weights, topk, expert_map,
                         num_global_experts, token_capacity, ws, size_t(MOE_STATIC_WORKSPACE_BYTES), out, stream);
}
