// Router epilogue: the fp32 logits (sum of K-chunk partials, chunk order
// fixed), softmax, top-k and renormalisation, one wavefront per token
// (Qwen3.8-Flash-Next study, MoE section: "Top 10 + normalize" in the
// pipeline figure; "Selected router probabilities are normalized").
//
// Each lane holds E/64 fp32 logits in registers.  k rounds of a wave-wide
// argmax (64-lane xor butterfly on (value, id), larger value wins, equal
// values go to the lower id) pick the experts in descending order; lane j
// keeps round j's winner.  The renormalised weight of the j-th pick is
// exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0), which equals the selected
// softmax probabilities divided by their sum (the full softmax's
// normaliser cancels).  Also the fp32 SIMT router used for fp32 layers.
#include <float.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <int PER_LANE>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int nsplit, int ldl, int T,
                                                   int E, int k, int has_sg, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, float* __restrict__ shared_logit) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // whole wave
  // logits = sum of the K-chunk partials, chunk order fixed
  const int64_t cstride = (int64_t)T * ldl;
  const float* row = partial + (int64_t)t * ldl;
  float v[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    float a = 0.f;
    if (e < E)
      for (int c = 0; c < nsplit; ++c) a += row[c * cstride + e];
    v[i] = e < E ? a : -FLT_MAX;
  }
  uint32_t taken = 0;
  float sel_v = 0.f;
  int sel_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
  }
  const float top = __shfl(sel_v, 0, 64);
  const float ex = lane < k ? expf(sel_v - top) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = sel_e;
    w[(int64_t)t * k + lane] = ex / sum;
  }
  if (has_sg && lane == 0) {
    float a = 0.f;
    for (int c = 0; c < nsplit; ++c) a += row[c * cstride + E];
    shared_logit[t] = a;
  }
}

// fp32 logits for fp32 layers: one thread per (token, column), h ascending.
__global__ void router_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr,
                                  const float* __restrict__ wsg, float* __restrict__ logits, int T, int H, int E,
                                  int N) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * N) return;
  const int t = (int)(idx / N), n = (int)(idx % N);
  const float* a = x + (int64_t)t * H;
  const float* b = n < E ? wr + (int64_t)n * H : wsg;
  float s = 0.f;
  for (int h = 0; h < H; ++h) s = fmaf(a[h], b[h], s);
  logits[idx] = s;
}

}  // namespace

hipError_t launch_topk(const float* partial, int nsplit, int ldl, int T, int E, int k, int has_sg, int32_t* ids,
                       float* w, float* shared_logit, hipStream_t s) {
  const int grid = (T + 3) / 4;
  const int per = (E + 63) / 64;
#define MOE_TOPK(P) topk_kernel<P><<<grid, 256, 0, s>>>(partial, nsplit, ldl, T, E, k, has_sg, ids, w, shared_logit)
  if (per <= 1) MOE_TOPK(1);
  else if (per <= 2) MOE_TOPK(2);
  else if (per <= 4) MOE_TOPK(4);
  else if (per <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

hipError_t launch_router_logits_f32(const float* x, const float* w_router, const float* w_sg, float* logits, int T,
                                    int H, int E, hipStream_t s) {
  const int N = E + (w_sg ? 1 : 0);
  const int64_t n = (int64_t)T * N;
  router_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, w_router, w_sg, logits, T, H, E, N);
  return hipGetLastError();
}

}  // namespace moe
