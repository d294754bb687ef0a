// moe_layer_forward_noalloc: the whole layer with its scratch in a
// file-scope device array, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops).  The array is part of
// the library's code object: each GPU the library runs on holds its own copy
// of MOE_NOALLOC_SCRATCH_BYTES bytes until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "kernels.hpp"
#include "moe_mi355x.h"

namespace moe {
namespace {

__device__ __attribute__((aligned(256))) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

// The device address of this GPU's copy of `scratch`.  The array's name is a
// host-side stand-in in host code, so its address is looked up once per
// device, with that device current, and only that address is handed to the
// kernels.  (Two threads racing on a device's first call look up the same
// address.)
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_layer_forward_noalloc(const moe_problem* p, const moe_weights* w, const void* x,
                                                 void* out, int32_t* topk_ids, float* topk_w, void* stream) {
  moe_status st = moe::layer_forward_checks(p, w, x, out);
  if (st != MOE_OK || p->T == 0) return st;
  if (moe_workspace_bytes(p) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if (moe::device_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
  // every launch on the caller's stream: no second stream is created here
  return moe::layer_forward_run(p, w, x, out, topk_ids, topk_w, ws, (hipStream_t)stream, /*fork_ok=*/false);
}
