// Dispatch (Qwen3.8-Flash-Next study, MoE section: the dispatch stage of its
// pipeline figure; its glance section defines R = 10T assignments, i.e. no
// drops): a stable counting sort of the R = T*k flat assignments
// a = t*k + j by expert id.
//
//  1. count  : one workgroup per chunk of 32 tokens; per-expert counts of
//              the chunk in LDS (LDS atomics only count, order comes later).
//  2. scan   : per expert, an exclusive scan of its chunk counts over the
//              chunks (64 experts per workgroup, chunks split over 16 waves)
//              and the expert's total.
//  3. scatter: one wave per chunk scans the E totals into expert_offsets,
//              then walks its tokens in order; lane j of a token takes its
//              expert's LDS cursor plus the number of lanes j' < j of the
//              same token with the same expert, and the last such lane
//              advances the cursor by the group's size, so positions come
//              out ascending in a within every expert (stable).
// The router never repeats an expert within a token (the layer call's
// dispatch skips the check), but moe_dispatch takes caller ids: a repeated id
// still gets its own slot (ordered by j), and ids outside [0, E) are clamped
// into range, so sorted_assign is always a permutation of [0, R) and
// assign_pos its inverse.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int CH = 32;  // tokens per chunk

__device__ __forceinline__ int clamp_e(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Lanes 0..k-1 of a wave hold the experts of one token.  For lane `lane`
// (< k): how many lanes before it hold the same expert, and how many hold it
// in all.  Lanes >= k pass e = -1, which matches no lane < k.  The lane index
// j of the readlane is uniform, so this is k scalar reads of e with no LDS
// round trip.
struct TokenRank {
  int before, group;
};
__device__ __forceinline__ TokenRank token_rank(int e, int lane, int k) {
  TokenRank r{0, 0};
  for (int j = 0; j < k; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    const int same = ej == e ? 1 : 0;
    r.group += same;
    r.before += j < lane ? same : 0;
  }
  return r;
}

// Wave-level scatter of up to CH consecutive tokens t0 .. t0+nt-1 in token
// order (lane j < k handles assignment a = t*k + j).  Every lane first loads
// its expert of every token.  Per token, each lane writes its lane index to
// mark[e] and reads it back: with no other lane of the token on e it reads
// its own index, so a mismatch anywhere means a repeated expert.  The router
// never repeats one, and then each lane takes p = cur[e], cur[e] = p + 1.
// Otherwise every lane adds its rank among the token's lanes with the same
// expert, and the last of them advances the cursor by the group's size.
template <bool CHECK>
__device__ __forceinline__ void scatter_tokens(const int32_t* __restrict__ ids, int t0, int nt, int E, int k,
                                               int lane, int* cur, int* mark, int32_t* __restrict__ sorted,
                                               int32_t* __restrict__ pos) {
  int ev[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i)
    ev[i] = (lane < k && i < nt) ? clamp_e(ids[(int64_t)(t0 + i) * k + lane], E) : -1;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (i < nt) {
      const int e = ev[i];
      const bool mine = lane < k;
      bool rep = false;
      if constexpr (CHECK) {
        // volatile: the read must observe the write instruction's winner, not
        // this lane's own stored value
        volatile int* mk = mark;
        if (mine) mk[e] = lane;
        rep = mine && mk[e] != lane;
      }
      const int64_t a = (int64_t)(t0 + i) * k + lane;
      if (__ballot(rep) == 0) {
        if (mine) {
          const int p = cur[e];
          cur[e] = p + 1;
          sorted[p] = (int32_t)a;
          pos[a] = p;
        }
      } else {
        const TokenRank rk = token_rank(e, lane, k);
        if (mine) {
          const int p = cur[e] + rk.before;
          if (rk.before + 1 == rk.group) cur[e] = p + 1;  // the token's last lane on e advances it
          sorted[p] = (int32_t)a;
          pos[a] = p;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

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

// Per expert, exclusive prefix of its chunk counts over chunks, in place, and
// the expert's total.  Block = 16 waves covering 64 experts (lane = expert);
// wave w owns a contiguous run of chunks, loads it with independent loads,
// then the 16 wave partials are scanned through LDS.
__global__ __launch_bounds__(1024) void chunk_scan_kernel(int32_t* __restrict__ chunk_counts, int nch, int E,
                                                          int32_t* __restrict__ totals) {
  __shared__ int part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int cpw = (nch + 15) / 16;
  const int c0 = w * cpw;
  const int c1 = c0 + cpw < nch ? c0 + cpw : nch;
  int sum = 0;
  if (e < E) {
    for (int c = c0; c < c1; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c + i < c1 ? chunk_counts[(int64_t)(c + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
  }
  part[w][lane] = sum;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < w; ++i) pre += part[i][lane];
  if (e < E) {
    if (w == 15) totals[e] = pre + sum;
    int run = pre;
    for (int c = c0; c < c1; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c + i < c1 ? chunk_counts[(int64_t)(c + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c + i < c1) chunk_counts[(int64_t)(c + i) * E + e] = run;
        run += v[i];
      }
    }
  }
}

// One wave per chunk.  The wave first turns the per-expert totals into
// expert offsets (every block redoes this small scan; block 0 publishes
// them), then walks its tokens in order: lane j of a token takes its
// expert's cursor plus its rank among the token's lanes with that expert.
template <bool CHECK>
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                     const int32_t* __restrict__ chunk_prefix,
                                                     const int32_t* __restrict__ totals,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                                     int32_t* __restrict__ pos) {
  extern __shared__ int cur[];  // [E] cursors, then [E] marks
  const int lane = threadIdx.x;
  // lane owns experts [lane*per, lane*per + per)
  const int per = (E + 63) / 64;
  const int e0 = lane * per;
  int local = 0;
  for (int i = 0; i < per; ++i) local += e0 + i < E ? totals[e0 + i] : 0;
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  int run = incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      if (blockIdx.x == 0) offsets[e] = run;
      cur[e] = run + chunk_prefix[(int64_t)blockIdx.x * E + e];
      run += totals[e];
    }
  }
  if (blockIdx.x == 0 && lane == 63) offsets[E] = incl;
  __syncthreads();
  const int t0 = blockIdx.x * CH;
  const int nt = T - t0 < CH ? T - t0 : CH;
  scatter_tokens<CHECK>(ids, t0, nt, E, k, lane, cur, cur + E, sorted, pos);
}

// Whole dispatch of a batch of at most CH tokens in one 1024-thread
// workgroup (decode): LDS counts, workgroup scan into expert_offsets, then
// wave 0 walks the tokens in order as in scatter_kernel.
template <bool CHECK>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted, int32_t* __restrict__ pos) {
  __shared__ int cur[1024];
  __shared__ int mark[1024];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  cur[tid] = 0;
  __syncthreads();
  const int R = T * k;
  for (int a = tid; a < R; a += blockDim.x) atomicAdd(&cur[clamp_e(ids[a], E)], 1);
  __syncthreads();
  const int v = tid < E ? cur[tid] : 0;
  const int lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[w] = incl;
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
  const int excl = incl - v + wsum[w];
  if (tid < E) {
    offsets[tid] = excl;
    cur[tid] = excl;
  }
  if (tid == 0) offsets[E] = R;
  __syncthreads();
  if (w == 0) scatter_tokens<CHECK>(ids, 0, T, E, k, lane, cur, mark, sorted, pos);
}

}  // namespace

size_t dispatch_ws_ints(int64_t T, int64_t E) { return (size_t)((T + CH - 1) / CH) * (size_t)E + (size_t)E; }

hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* sorted,
                           int32_t* pos, int32_t* ws, hipStream_t s, bool distinct) {
  if (T <= CH) {
    if (distinct) dispatch_small_kernel<false><<<1, 1024, 0, s>>>(ids, T, E, k, offsets, sorted, pos);
    else dispatch_small_kernel<true><<<1, 1024, 0, s>>>(ids, T, E, k, offsets, sorted, pos);
    return hipGetLastError();
  }
  const int nch = (T + CH - 1) / CH;
  int32_t* totals = ws + (size_t)nch * E;
  count_kernel<<<nch, 256, E * sizeof(int), s>>>(ids, T, E, k, ws);
  chunk_scan_kernel<<<(E + 63) / 64, 1024, 0, s>>>(ws, nch, E, totals);
  if (distinct) scatter_kernel<false><<<nch, 64, 2 * E * sizeof(int), s>>>(ids, T, E, k, ws, totals, offsets, sorted, pos);
  else scatter_kernel<true><<<nch, 64, 2 * E * sizeof(int), s>>>(ids, T, E, k, ws, totals, offsets, sorted, pos);
  return hipGetLastError();
}

}  // namespace moe
