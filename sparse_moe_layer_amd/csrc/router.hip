// Router epilogue: the fp32 logits (sum of K-chunk partials, chunk order
// fixed), softmax, top-k and renormalisation, one wavefront per token
// (Qwen3.8-Flash-Next study, MoE section: the top-k stage of its pipeline
// figure, where the chosen experts' probabilities are renormalised to sum to
// one).
//
// Each lane holds E/64 logits as 64-bit keys: an order-preserving image of
// the fp32 value in the high word, the complement of the expert id in the low
// word, so one unsigned maximum ranks by value and sends equal values to the
// lower id.  k rounds of a wave-wide maximum (DPP within each 16-lane row,
// then the four row results through readlane) pick the experts in descending
// order; lane j keeps round j's winner.  The renormalised weight of the j-th
// pick is exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0), which equals the
// selected softmax probabilities divided by their sum (the full softmax's
// normaliser cancels).  With the section's routing numerics for bf16 layers
// the logits are rounded to bf16 first (ties become common) and the weights
// are rounded to bf16 last.  Also the fp32 SIMT router used for fp32 layers.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Monotone map fp32 -> u32 (a < b as floats <=> ord(a) < ord(b) unsigned),
// with -0 folded onto +0 so that equal values compare equal.  Every real
// logit maps above 0, which marks padding and taken entries.
__device__ __forceinline__ uint32_t ord(float v) {
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord(uint32_t m) { return __uint_as_float((m >> 31) ? (m & 0x7fffffffu) : ~m); }

__device__ __forceinline__ void key_max(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
  const bool gt = ohi > hi || (ohi == hi && olo > lo);
  hi = gt ? ohi : hi;
  lo = gt ? olo : lo;
}

template <int CTRL>
__device__ __forceinline__ void dpp_max(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, 0xf, 0xf, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, 0xf, 0xf, false);
  key_max(hi, lo, ohi, olo);
}

// Maximum key over the 64 lanes, returned in every lane.
__device__ __forceinline__ void wave_key_max(uint32_t& hi, uint32_t& lo) {
  dpp_max<0xb1>(hi, lo);   // quad_perm [1,0,3,2]
  dpp_max<0x4e>(hi, lo);   // quad_perm [2,3,0,1]: quad maximum in every lane
  dpp_max<0x141>(hi, lo);  // row_half_mirror: 8-lane maximum
  dpp_max<0x140>(hi, lo);  // row_mirror: 16-lane (row) maximum
  uint32_t bh = __builtin_amdgcn_readlane(hi, 0), bl = __builtin_amdgcn_readlane(lo, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    key_max(bh, bl, __builtin_amdgcn_readlane(hi, 16 * r), __builtin_amdgcn_readlane(lo, 16 * r));
  hi = bh;
  lo = bl;
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int nsplit, int ldl, int T,
                                                   int E, int k, int has_sg, int page, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, float* __restrict__ shared_logit) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;  // whole wave
  // logits = sum of the K-chunk partials, chunk order fixed
  const int64_t cstride = (int64_t)T * ldl;
  const float* row = partial + (int64_t)t * ldl;
  uint32_t khi[PER_LANE], klo[PER_LANE];
  float lg[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) lg[i] = 0.f;
  // four chunks at a time, the loads of all of this lane's logits in flight
  // together, then added in chunk order
  for (int c0 = 0; c0 < nsplit; c0 += 4) {
    float v[4][PER_LANE];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i;
        v[u][i] = (c0 + u < nsplit && e < E) ? row[(c0 + u) * cstride + e] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i)
        if (c0 + u < nsplit) lg[i] += v[u][i];
  }
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    float a = lg[i];
    if (page) a = bf2f(f2bf(a));  // logits in the activation dtype (round to nearest even)
    khi[i] = e < E ? ord(a) : 0u;
    klo[i] = ~(uint32_t)e;
  }
  uint32_t sel_hi = 0, sel_lo = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t bh = khi[0], bl = klo[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) key_max(bh, bl, khi[i], klo[i]);
    wave_key_max(bh, bl);
    const int e = (int)~bl;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + 64 * i == e) khi[i] = 0u;  // taken
    if (lane == j) {
      sel_hi = bh;
      sel_lo = bl;
    }
  }
  const float top = unord(__builtin_amdgcn_readlane(sel_hi, 0));
  const float ex = lane < k ? expf(unord(sel_hi) - top) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    const float wj = ex / sum;
    ids[(int64_t)t * k + lane] = (int32_t)~sel_lo;
    w[(int64_t)t * k + lane] = page ? bf2f(f2bf(wj)) : wj;  // mixing weight in the activation dtype
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

hipError_t launch_topk(const float* partial, int nsplit, int ldl, int T, int E, int k, int has_sg, bool page,
                       int32_t* ids, float* w, float* shared_logit, hipStream_t s) {
  const int grid = (T + 3) / 4;
  const int per = (E + 63) / 64;
#define MOE_TOPK(P) \
  topk_kernel<P><<<grid, 256, 0, s>>>(partial, nsplit, ldl, T, E, k, has_sg, page ? 1 : 0, ids, w, shared_logit)
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
