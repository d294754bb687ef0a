// Dispatch (Qwen3.8-Flash-Next study, MoE section: "Dispatch R tokens"; the
// glance section defines R = 10T assignments, i.e. no drops): a stable
// counting sort of the R = T*k flat assignments a = t*k + j by expert id.
//
//  1. count  : one workgroup per chunk of 32 tokens; per-expert counts of
//              the chunk in LDS (LDS atomics only count, order comes later).
//  2. scan   : one 1024-thread workgroup; for every expert an exclusive scan
//              over chunks, then a workgroup scan of the per-expert totals
//              gives expert_offsets; chunk bases = offset + prefix.
//  3. scatter: one wave per chunk walks its tokens in order; the k lanes of
//              a token hit k distinct experts, so each lane bumps its expert's
//              LDS cursor without conflict, and positions come out ascending
//              in a within every expert (stable).
// Expert ids outside [0, E) are clamped into range so the result is always a
// permutation (memory-safe); ids repeated within a token give an
// unspecified (still in-range) order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int CH = 32;  // tokens per chunk

__device__ __forceinline__ int clamp_e(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                    int32_t* __restrict__ chunk_counts) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * CH * k;
  int64_t a1 = a0 + (int64_t)CH * k;
  const int64_t R = (int64_t)T * k;
  a1 = a1 < R ? a1 : R;
  for (int64_t a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&cnt[clamp_e(ids[a], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ chunk_counts, int nch, int E, int R,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  // per-expert exclusive scan over chunks (E <= 1024: one expert per thread)
  int run = 0;
  if (tid < E) {
    for (int c = 0; c < nch; ++c) {
      int32_t* p = chunk_counts + (int64_t)c * E + tid;
      const int v = *p;
      *p = run;
      run += v;
    }
  }
  // workgroup exclusive scan of totals
  const int lane = tid & 63, w = tid >> 6;
  int s = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(s, o, 64);
    if (lane >= o) s += t;
  }
  if (lane == 63) wsum[w] = s;
  __syncthreads();
  if (w == 0) {
    const int t = lane < 16 ? wsum[lane] : 0;
    int u = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int q = __shfl_up(u, o, 64);
      if (lane >= o) u += q;
    }
    if (lane < 16) wsum[lane] = u - t;
  }
  __syncthreads();
  const int excl = s - run + wsum[w];
  if (tid < E) offsets[tid] = excl;
  if (tid == 0) offsets[E] = R;
  __syncthreads();
  if (tid < E) {
    for (int c = 0; c < nch; ++c) chunk_counts[(int64_t)c * E + tid] += excl;
  }
}

__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                     const int32_t* __restrict__ chunk_base,
                                                     int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  extern __shared__ int cur[];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) cur[e] = chunk_base[(int64_t)blockIdx.x * E + e];
  __syncthreads();
  const int t0 = blockIdx.x * CH;
  const int t1 = t0 + CH < T ? t0 + CH : T;
  for (int t = t0; t < t1; ++t) {
    if (lane < k) {
      const int64_t a = (int64_t)t * k + lane;
      const int e = clamp_e(ids[a], E);
      const int p = cur[e];
      cur[e] = p + 1;
      sorted[p] = (int32_t)a;
      pos[a] = p;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

size_t dispatch_ws_ints(int64_t T, int64_t E) { return (size_t)((T + CH - 1) / CH) * (size_t)E; }

hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* sorted,
                           int32_t* pos, int32_t* ws, hipStream_t s) {
  const int nch = (T + CH - 1) / CH;
  count_kernel<<<nch, 256, E * sizeof(int), s>>>(ids, T, E, k, ws);
  scan_kernel<<<1, 1024, 0, s>>>(ws, nch, E, T * k, offsets);
  scatter_kernel<<<nch, 64, E * sizeof(int), s>>>(ids, T, E, k, ws, sorted, pos);
  return hipGetLastError();
}

}  // namespace moe
