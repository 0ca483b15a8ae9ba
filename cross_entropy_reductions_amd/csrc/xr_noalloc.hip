// xr_noalloc.hip -- the fused cross-entropy for callers that cannot allocate: its scratch is
// a static device array of the library instead of a caller's workspace.
//
// `scratch` below is one array per device (each device that loads the library's code object
// gets its own copy). In host code its name is only a stand-in for the symbol, never a
// device address: the address is looked up once per device, with that device current,
// through hipGetSymbolAddress, and only that address is passed on.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "../../include/xr.h"

namespace {

constexpr size_t kScratchBytes = XR_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> that device's copy of `scratch`

// The current device's copy of `scratch` (looked up on the first call on that device).
xr_status_t current_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return XR_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return XR_ERR_DEVICE;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return XR_OK;
}

}  // namespace

extern "C" xr_status_t xr_xent_fwd_bwd_noalloc(void* logits, int64_t ld, const int64_t* target,
                                               int64_t M, int64_t V, int64_t ignore_index,
                                               xr_dtype_t dtype, xr_reduction_t reduction,
                                               const float* grad_scale, int64_t grad_scale_stride,
                                               float* row_loss, float* loss, int32_t* counts,
                                               void* stream) {
  void* ws = nullptr;
  if (xr_status_t st = current_scratch(&ws)) return st;
  // The workspace entry point validates everything and checks the scratch's size against
  // the plan before it enqueues anything; the scratch is never NULL, so a workspace error
  // can only mean the sizes need more scratch than the array holds.
  const xr_status_t st =
      xr_xent_fwd_bwd_ex(logits, ld, target, M, V, ignore_index, dtype, reduction, grad_scale,
                         grad_scale_stride, row_loss, loss, counts, ws, kScratchBytes, stream);
  return st == XR_ERR_WORKSPACE ? XR_ERR_TOO_LARGE : st;
}
