// The whole routed layer without a caller workspace: moe_layer_noalloc.
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The
// layer's scratch -- logits, router group sums, permutation, tile plan,
// SwiGLU intermediate and expert outputs -- lives in the file-scope device
// array below instead of a workspace argument.  Each device the library runs
// on holds its own copy of the array (MOE_NOALLOC_SCRATCH_BYTES) from the
// first use until the process ends.
//
// The array's name in host code is only a host-side stand-in for the
// symbol; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, guarded by the mutex

// ScratchFn of moe_layer_noalloc: the size limit first (host-only, so an
// oversized call is rejected before any HIP call), then the array of the
// stream's device, which must be the current device.
int static_scratch(size_t need, hipStream_t st, void** ws, size_t* ws_bytes) {
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_E_WORKSPACE;
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &sdev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_E_DEVICE;
  }
  if (cur < 0 || cur >= kMaxDevices || sdev != cur) return MOE_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MOE_E_DEVICE;
    }
    g_scratch_ptr[cur] = p;
  }
  *ws = g_scratch_ptr[cur];
  *ws_bytes = MOE_NOALLOC_SCRATCH_BYTES;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_layer_noalloc(const moe_shape* shape, const void* x, const void* w_router,
                                 const float* router_bias, const moe_experts* experts,
                                 const void* residual, void* out, int32_t* topk_ids, float* topk_w,
                                 const moe_perm* perm, hipStream_t stream) {
  return moe::layer_call(shape, x, w_router, router_bias, experts, residual, out, topk_ids, topk_w,
                         perm, nullptr, 0, stream, moe::static_scratch);
}
