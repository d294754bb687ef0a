// moe_hbm_read_probe: reads a buffer once with the access the streaming
// kernels use at their best (16 bytes per lane, whole waves on contiguous
// runs, several loads in flight per lane) and nothing else, so its rate is
// the practical HBM read ceiling the streaming rooflines are read against.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "moe_mi355x.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeDepth = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                     uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (kProbeDepth - 1) * stride < n16; i += kProbeDepth * stride) {
    u32x4 v[kProbeDepth];
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) v[d] = __builtin_nontemporal_load(src + i + d * stride);
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) acc ^= v[d];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) sink[0] = r;  // keeps the loads; practically never taken
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || bytes % 16) return MOE_ERR_ALIGN;
  if (bytes == 0) return MOE_OK;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOE_ERR_HIP;
  const int64_t n16 = (int64_t)(bytes / 16);
  moe::hbm_read_probe_kernel<<<cus * 8, moe::kProbeThreads, 0, (hipStream_t)stream>>>(
      static_cast<const moe::u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
