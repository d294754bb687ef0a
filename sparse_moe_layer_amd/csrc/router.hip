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

// Keys: the order-preserving image of the logit in the high word, the
// complement of the expert id in the low word; one unsigned 64-bit maximum
// ranks by value and sends equal values to the lower id.
__device__ __forceinline__ uint64_t make_key(uint32_t ordv, int e) { return ((uint64_t)ordv << 32) | (uint32_t)~e; }
__device__ __forceinline__ uint64_t key_max(uint64_t a, uint64_t b) { return b > a ? b : a; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, 0xf, 0xf, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, 0xf, 0xf, false);
  return key_max(k, ((uint64_t)ohi << 32) | olo);
}

// Maximum key over the 64 lanes (wave-uniform result).
__device__ __forceinline__ uint64_t wave_key_max(uint64_t k) {
  k = dpp_max<0xb1>(k);   // quad_perm [1,0,3,2]
  k = dpp_max<0x4e>(k);   // quad_perm [2,3,0,1]: quad maximum in every lane
  k = dpp_max<0x141>(k);  // row_half_mirror: 8-lane maximum
  k = dpp_max<0x140>(k);  // row_mirror: 16-lane (row) maximum
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  uint64_t b = make_key(0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    // (readlane returns int: widen through uint32_t, not by sign extension)
    const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane(lo, 16 * r);
    b = r == 0 ? o : key_max(b, o);
  }
  return b;
}

template <int PER_LANE>
__device__ __forceinline__ void token_topk(const float* __restrict__ partial, int nsplit, int ldl, int T, int E,
                                           int k, int has_sg, int page, int t, int lane, int32_t* __restrict__ ids,
                                           float* __restrict__ w, float* __restrict__ shared_logit, int* lds_ids) {
  // logits = sum of the K-chunk partials, chunk order fixed
  const int64_t cstride = (int64_t)T * ldl;
  const float* row = partial + (int64_t)t * ldl;
  uint64_t key[PER_LANE];
  float lg[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) lg[i] = 0.f;
  // four chunks at a time, every load unconditional (addresses clamped into
  // the row, padding lanes zeroed later), then added in chunk order
  for (int c0 = 0; c0 < nsplit; c0 += 4) {
    float v[4][PER_LANE];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u < nsplit ? c0 + u : nsplit - 1;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        const int e = lane + 64 * i < E ? lane + 64 * i : E - 1;
        v[u][i] = row[c * cstride + e];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + u < nsplit)
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) lg[i] += v[u][i];
  }
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + 64 * i;
    float a = lg[i];
    if (page) a = bf2f(f2bf(a));  // logits in the activation dtype (round to nearest even)
    key[i] = make_key(e < E ? ord(a) : 0u, e);
  }
  // each lane's keys in descending order (odd-even transposition sort), so
  // a round only compares the 64 lane heads and pops the winner's head
#pragma unroll
  for (int r = 0; r < PER_LANE; ++r)
#pragma unroll
    for (int i = r & 1; i + 1 < PER_LANE; i += 2) {
      const uint64_t a = key[i], b = key[i + 1];
      key[i] = key_max(a, b);
      key[i + 1] = b > a ? a : b;
    }
  uint64_t sel = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t b = wave_key_max(key[0]);
    // the winner (one lane: keys are unique) pops its head; a bit mask
    // rather than a select, which the compiler would turn into an indexed
    // read of the key array
    const uint64_t m = key[0] == b ? ~0ull : 0ull;
#pragma unroll
    for (int i = 0; i + 1 < PER_LANE; ++i) key[i] = (key[i + 1] & m) | (key[i] & ~m);
    key[PER_LANE - 1] &= ~m;
    if (lane == j) sel = b;
  }
  const uint32_t sel_hi = (uint32_t)(sel >> 32), sel_lo = (uint32_t)sel;
  const float top = unord(__builtin_amdgcn_readlane(sel_hi, 0));
  const float ex = lane < k ? expf(unord(sel_hi) - top) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    const float wj = ex / sum;
    ids[(int64_t)t * k + lane] = (int32_t)~sel_lo;
    w[(int64_t)t * k + lane] = page ? bf2f(f2bf(wj)) : wj;  // mixing weight in the activation dtype
    if (lds_ids) lds_ids[t * k + lane] = (int)~sel_lo;
  }
  if (has_sg && lane == 0) {
    float a = 0.f;
    for (int c = 0; c < nsplit; ++c) a += row[c * cstride + E];
    shared_logit[t] = a;
  }
}

template <int PER_LANE>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partial, int nsplit, int ldl, int T,
                                                   int E, int k, int has_sg, int page, int32_t* __restrict__ ids,
                                                   float* __restrict__ w, float* __restrict__ shared_logit) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  token_topk<PER_LANE>(partial, nsplit, ldl, T, E, k, has_sg, page, t, threadIdx.x & 63, ids, w, shared_logit,
                       nullptr);
}

// Top-k and dispatch of a batch of at most kSmallBatch tokens in one kernel:
// workgroup t (one wave) picks token t's experts as topk_kernel does; the
// last workgroup to finish (a device-scope counter, zero at launch) then
// performs the dispatch of the section's pipeline figure for the whole
// batch: a bit mask per expert of the tokens that chose it (a token's k
// picks are distinct experts), an exclusive scan of the mask populations
// into expert_offsets, and each assignment a = t*k + j placed at its
// expert's offset plus the number of earlier tokens in the expert's mask,
// which is its rank among the expert's assignments in ascending a: the same
// stable order as the counting sort of the dispatch kernels.  The last
// workgroup leaves the counter at zero.
template <int PER_LANE>
__global__ __launch_bounds__(64) void topk_dispatch_small_kernel(
    const float* __restrict__ partial, int nsplit, int ldl, int T, int E, int k, int has_sg, int page,
    int32_t* __restrict__ ids, float* __restrict__ w, float* __restrict__ shared_logit, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ pos, int32_t* counter) {
  __shared__ uint32_t mask[kMaxExperts];
  __shared__ int start[kMaxExperts];
  const int lane = threadIdx.x;
  token_topk<PER_LANE>(partial, nsplit, ldl, T, E, k, has_sg, page, blockIdx.x, lane, ids, w, shared_logit,
                       nullptr);
  __threadfence();  // this token's ids are visible device-wide before it is counted
  int last = 0;
  if (lane == 0) last = atomicAdd(counter, 1) == T - 1 ? 1 : 0;
  if (!__builtin_amdgcn_readfirstlane(last)) return;
  __threadfence();  // every token's ids are visible here
  const int R = T * k;
  for (int e = lane; e < E; e += 64) mask[e] = 0u;
  __syncthreads();
  for (int a = lane; a < R; a += 64) atomicOr(&mask[ids[a]], 1u << (a / k));
  __syncthreads();
  // exclusive scan of the populations: lane owns experts [lane*per, +per)
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int local = 0;
  for (int i = 0; i < per; ++i) local += e0 + i < E ? __popc(mask[e0 + i]) : 0;
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  int run = incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      offsets[e] = run;
      start[e] = run;
      run += __popc(mask[e]);
    }
  }
  if (lane == 63) offsets[E] = incl;
  __syncthreads();
  for (int a = lane; a < R; a += 64) {
    const int e = ids[a];
    const int t = a / k;
    const int p = start[e] + __popc(mask[e] & ((1u << t) - 1u));
    sorted[p] = a;
    pos[a] = p;
  }
  if (lane == 0) *counter = 0;
}

// fp32 logits for fp32 layers: one thread per (token, column), h ascending.
__global__ void router_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr,
                                  const float* __restrict__ wsg, float* __restrict__ logits, int T, int H, int E,
                                  int N, int32_t* zero_word) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (zero_word && idx == 0) *zero_word = 0;  // a word the next kernel needs at zero (or null)
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

hipError_t launch_topk_dispatch_small(const float* partial, int nsplit, int ldl, int T, int E, int k, int has_sg,
                                     bool page, int32_t* ids, float* w, float* shared_logit, int32_t* offsets,
                                     int32_t* sorted, int32_t* pos, int32_t* counter, hipStream_t s) {
  if (T < 1 || T > kSmallBatch || k > 64 || E > kMaxExperts || !counter) return hipErrorInvalidValue;
  const int per = (E + 63) / 64;
#define MOE_TOPK_DISPATCH(P)                                                                                    \
  topk_dispatch_small_kernel<P><<<T, 64, 0, s>>>(partial, nsplit, ldl, T, E, k, has_sg, page ? 1 : 0, ids, w, \
                                                 shared_logit, offsets, sorted, pos, counter)
  if (per <= 1) MOE_TOPK_DISPATCH(1);
  else if (per <= 2) MOE_TOPK_DISPATCH(2);
  else if (per <= 4) MOE_TOPK_DISPATCH(4);
  else if (per <= 8) MOE_TOPK_DISPATCH(8);
  else MOE_TOPK_DISPATCH(16);
#undef MOE_TOPK_DISPATCH
  return hipGetLastError();
}

hipError_t launch_router_logits_f32(const float* x, const float* w_router, const float* w_sg, float* logits, int T,
                                    int H, int E, hipStream_t s, int32_t* zero_word) {
  const int N = E + (w_sg ? 1 : 0);
  const int64_t n = (int64_t)T * N;
  router_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(x, w_router, w_sg, logits, T, H, E, N, zero_word);
  return hipGetLastError();
}

}  // namespace moe
