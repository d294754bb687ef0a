// Expert FFN for fp32 layers (all tensors fp32): plain SIMT dot products, one
// thread per output element, K ascending.  Covers small fp32 layers only;
// bf16/fp8 layers run on the MFMA kernels.  Same math as eq. expert(x) in
// the Qwen3.8-Flash-Next study's MoE section.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// expert owning dispatched row r: last e with offsets[e] <= r
__device__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // invariant offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// rows [0, R) routed, rows [R, R+T) shared (when present)
__global__ void gateup_f32(FfnArgs f, int R, int rows) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int wide = f.I > f.Is ? f.I : f.Is;
  if (idx >= (int64_t)rows * wide) return;
  const int r = (int)(idx / wide), j = (int)(idx % wide);
  const float* x = reinterpret_cast<const float*>(f.x);
  const float *wg, *wu, *a;
  float* dst;
  if (r < R) {
    if (j >= f.I) return;
    const int e = expert_of_row(f.offsets, f.E, r);
    int tok = f.sorted[r] / f.k;
    tok = (unsigned)tok < (unsigned)f.T ? tok : f.T - 1;  // also clamps a negative index
    a = x + (int64_t)tok * f.H;
    wg = reinterpret_cast<const float*>(f.wg) + (int64_t)e * f.sg + (int64_t)j * f.H;
    wu = reinterpret_cast<const float*>(f.wu) + (int64_t)e * f.su + (int64_t)j * f.H;
    dst = reinterpret_cast<float*>(f.h) + (int64_t)r * f.I + j;
  } else {
    if (j >= f.Is) return;
    const int t = r - R;
    a = x + (int64_t)t * f.H;
    wg = reinterpret_cast<const float*>(f.shg) + (int64_t)j * f.H;
    wu = reinterpret_cast<const float*>(f.shu) + (int64_t)j * f.H;
    dst = reinterpret_cast<float*>(f.h_sh) + (int64_t)t * f.Is + j;
  }
  float g = 0.f, u = 0.f;
  for (int h = 0; h < f.H; ++h) {
    g = fmaf(a[h], wg[h], g);
    u = fmaf(a[h], wu[h], u);
  }
  *dst = silu(g) * u;
}

__global__ void down_f32(FfnArgs f, int R, int rows) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * f.H) return;
  const int r = (int)(idx / f.H), n = (int)(idx % f.H);
  const float *a, *wd;
  float* dst;
  int K;
  if (r < R) {
    const int e = expert_of_row(f.offsets, f.E, r);
    a = reinterpret_cast<const float*>(f.h) + (int64_t)r * f.I;
    wd = reinterpret_cast<const float*>(f.wd) + (int64_t)e * f.sd + (int64_t)n * f.I;
    dst = reinterpret_cast<float*>(f.y) + (int64_t)r * f.H + n;
    K = f.I;
  } else {
    const int t = r - R;
    a = reinterpret_cast<const float*>(f.h_sh) + (int64_t)t * f.Is;
    wd = reinterpret_cast<const float*>(f.shd) + (int64_t)n * f.Is;
    dst = reinterpret_cast<float*>(f.y_sh) + (int64_t)t * f.H + n;
    K = f.Is;
  }
  float s = 0.f;
  for (int i = 0; i < K; ++i) s = fmaf(a[i], wd[i], s);
  *dst = s;
}

}  // namespace

hipError_t launch_ffn_f32(const FfnArgs& a, int phases, hipStream_t s) {
  const int R = a.T * a.k;
  const int rows = R + (a.Is > 0 ? a.T : 0);
  const int wide = a.I > a.Is ? a.I : a.Is;
  const int64_t n1 = (int64_t)rows * wide, n2 = (int64_t)rows * a.H;
  if ((phases & 1) && n1 > 0) gateup_f32<<<(unsigned)((n1 + 255) / 256), 256, 0, s>>>(a, R, rows);
  if ((phases & 2) && n2 > 0) down_f32<<<(unsigned)((n2 + 255) / 256), 256, 0, s>>>(a, R, rows);
  return hipGetLastError();
}

}  // namespace moe
