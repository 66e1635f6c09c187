// The MoE forward pass for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the same launches as moe_mxfp4_forward, on
// a workspace that is a file-scope device array of MXFP4_NOALLOC_SCRATCH_BYTES instead of a caller
// buffer.  Each device the library runs on holds its own copy of the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is taken
// once per device with hipGetSymbolAddress (with that device current, on the first call made there)
// and only that address is handed to the kernels.  Every call on a device shares the array and finds
// what the last call left in it; the forward pass clears what must start at zero (the routing
// histogram) with a kernel of its own, so no memset is involved.  Calls that overlap on one device
// (on different streams without ordering between them) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

#define MX_API extern "C" __attribute__((visibility("default")))

namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's copy of the array, or NULL if it cannot be had.
void* scratch_address(int dev) {
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_dev[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
  });
  return g_scratch_dev[dev];
}

}  // namespace

MX_API int moe_mxfp4_forward_noalloc(const mxfp4_moe_dims* d, const void* packed_gfx950, const void* x_bf16, int64_t T,
                                     int64_t ldx, const float* router_logits, int32_t top_k, int32_t renormalize,
                                     void* y_bf16, int32_t* topk_ids, float* topk_w, void* stream) {
  const size_t need = moe_mxfp4_workspace_bytes(d, T, top_k);
  // argument errors, or no tokens: the status of the same call on a caller workspace, and no device
  // contact
  if (need == 0 || T == 0)
    return forward_impl(d, MXFP4_ACT_BF16, packed_gfx950, x_bf16, T, ldx, router_logits, top_k, renormalize, y_bf16,
                        topk_ids, topk_w, nullptr, 0, (hipStream_t)stream, nullptr, 0);
  if (need > (size_t)MXFP4_NOALLOC_SCRATCH_BYTES) return MXFP4_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXFP4_ERR_DEVICE;
  void* ws = scratch_address(dev);
  if (!ws) return MXFP4_ERR_DEVICE;
  return forward_impl(d, MXFP4_ACT_BF16, packed_gfx950, x_bf16, T, ldx, router_logits, top_k, renormalize, y_bf16,
                      topk_ids, topk_w, ws, (size_t)MXFP4_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream, nullptr, 0);
}
