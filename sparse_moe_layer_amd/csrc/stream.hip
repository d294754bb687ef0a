// Weight-streaming kernels for groups with few rows (decode, skew tails) and
// the split-K router for small batches.
//
// When an expert holds only a handful of tokens the expert GEMMs of
// eq. expert(x) (Qwen3.8-Flash-Next study, MoE section) are bound by reading
// its weights once from HBM.  Each wave owns one (16-row m-block, weight slab)
// item (stream_item.hpp) and streams the slab's weight rows once from HBM
// (every weight byte is used by exactly one wave).  HBM wants long runs per
// row: a fragment-shaped load touches 16 rows x 64 B and runs at well under
// half the bandwidth of 512-byte runs, so bf16 weights are loaded in 512-byte
// runs and fp8 codes in 256-byte runs.
//   router item : 16 router rows (the shared-gate row last) over one K chunk,
//                 fp32 partial logits, reduced in fixed order by the top-k kernel
#include "common.hpp"
#include "kernels.hpp"
#include "stream_item.hpp"

namespace moe {
namespace {

using namespace streamk;
constexpr int WAVES = 4;

// acc[j] += A[16 rows, kbeg..kend) x B_j[16 rows, kbeg..kend)^T for NB bf16
// weight blocks, operands loaded straight into MFMA fragments (the small-batch
// router).  a_row: this lane's A row (row lane%16) or null (zero row);
// b_row[j]: this lane's row of weight block j.  kq = 8*(lane/16) is the
// lane's K offset inside a 32-wide K step.  U K steps per batch, two batches
// in flight.
template <int NB>
__device__ __forceinline__ void stream_dot(const bf16* a_row, const bf16* const* b_row, int kbeg, int kend, int kq,
                                           f32x4* acc) {
  u32x4 av[2][U];
  u32x4 bv[2][U][NB];
  const int nsteps = (kend - kbeg + KSTEP - 1) / KSTEP;
  auto load = [&](int buf, int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = kbeg + (s0 + u) * KSTEP + kq;
      const bool in = kk < kend;
      av[buf][u] = (in && a_row) ? ld16(a_row + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[buf][u][j] = in ? ld16(b_row[j] + kk) : u32x4{0, 0, 0, 0};
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[buf][u]), as_bf16x8(bv[buf][u][j]), acc[j],
                                                         0, 0, 0);
  };
  load(0, 0);
  for (int s0 = 0; s0 < nsteps; s0 += 2 * U) {
    const bool more = s0 + U < nsteps;
    if (more) load(1, s0 + U);
    mma(0);
    if (more) {
      if (s0 + 2 * U < nsteps) load(0, s0 + 2 * U);
      mma(1);
    }
  }
}

// SPLIT (bf16 gate/up only): items of 8 hidden columns, one 16-row block of
// 8 gate rows and the 8 up rows of the same columns.  Half-size items end a
// launch with less idle time; they pay off when the whole batch streams
// (decode) and cost a few percent on large streaming tails, where 16-column
// items (a 16-row gate block and a 16-row up block) keep more bytes in
// flight per wave.  Down items are 32 output columns (2 blocks).
//
// SELF_PLAN (batches of at most kStreamMaxRows tokens, where every group
// streams as one m-block): no plan kernel runs before the launch; each
// workgroup lists the touched groups itself, in ascending order with the
// shared expert last, from the expert offsets (the plan's stream list for
// such a batch); the list bounds name plan positions as without it.
// self_plan == 2 (route.ids non-null; bf16 gate/up split items, T <=
// kSmallBatch): the dispatch is not in memory yet.  Each workgroup ORs every
// assignment a = t*k + j into its expert's token mask in LDS (bit t; a
// token's picks are distinct experts), lists the experts with a nonzero mask
// as (expert | mask << 11), and takes an item's first dispatched row as the
// number of rows of the experts listed before it: the stable order of the
// dispatch kernels, in which an expert's rows are its tokens ascending.
// Wave 0 of workgroup 0 also writes offsets, sorted and pos from the masks.
template <int PHASE, bool FP8, bool SPLIT = false>
__global__ __launch_bounds__(WAVES * 64, 2) void stream_kernel(FfnArgs f, int list_begin_idx, int list_end_idx,
                                                               int self_plan, SmallRoute route) {
  static_assert(!SPLIT || (PHASE == 1 && !FP8), "split items are bf16 gate/up");
  constexpr int STAGE_BYTES = item_lds_bytes<FP8, SPLIT>();  // per wave
  constexpr bool ROUTES = PHASE == 1 && !FP8 && SPLIT;       // may take the dispatch (self_plan == 2)
  // the masks and (workgroup 0) the experts' first rows fit wave 0's own stage buffer
  static_assert(!ROUTES || 2 * kMaxExperts * 4 <= STAGE_BYTES, "route scratch in the stage");
  __shared__ __attribute__((aligned(16))) char stage[WAVES * STAGE_BYTES];
  __shared__ int glist[kMaxExperts + 1];  // SELF_PLAN: touched groups
  __shared__ int wtot[WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int nw = gridDim.x * WAVES;
  int sb_begin, sb_end;
  // route: token masks per expert in the stage buffers until the items start
  uint32_t* tmask = reinterpret_cast<uint32_t*>(stage);
  const bool routed = ROUTES && self_plan == 2;
  if (routed) {
    for (int e = threadIdx.x; e < f.E; e += WAVES * 64) tmask[e] = 0u;
    __syncthreads();
    for (int a = threadIdx.x; a < f.T * f.k; a += WAVES * 64) {
      int e = route.ids[a];
      e = (unsigned)e < (unsigned)f.E ? e : f.E - 1;  // (the router's ids are in range)
      atomicOr(&tmask[e], 1u << (a / f.k));
    }
    __syncthreads();
  }
  if (self_plan) {
    // ordered compaction of the routed groups with rows, 64*WAVES at a time:
    // a wave's ballot gives each lane its rank, the waves' totals its offset
    int n_routed = 0;
    for (int g0 = 0; g0 < f.E; g0 += WAVES * 64) {
      const int g = g0 + threadIdx.x;
      uint32_t mk = 0u;
      bool t;
      if (routed) {
        mk = g < f.E ? tmask[g] : 0u;
        t = mk != 0u;
      } else {
        t = g < f.E && f.offsets[g + 1] > f.offsets[g];
      }
      const uint64_t bal = __ballot(t);
      const int rank = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[wave] = __popcll(bal);
      __syncthreads();
      int off = n_routed;
      for (int w = 0; w < wave; ++w) off += wtot[w];
      if (t) glist[off + rank] = routed ? (int)((uint32_t)g | (mk << 11)) : g;
      for (int w = 0; w < WAVES; ++w) n_routed += wtot[w];
      __syncthreads();
    }
    if (threadIdx.x == 0) glist[n_routed] = f.E;  // the shared expert (read only when present)
    __syncthreads();
    if (routed && blockIdx.x == 0 && wave == 0) {
      // the dispatch's outputs: offsets from an exclusive scan of the mask
      // populations (lane i owns experts [i*per, (i+1)*per)), then each
      // assignment at its expert's first row plus its token's rank in the
      // expert's mask.  The start of each expert goes to the second half of
      // the scratch (this wave's own stage buffer, before its items).
      int* start = reinterpret_cast<int*>(tmask + kMaxExperts);
      const int per = (f.E + 63) / 64;
      const int e0 = lane * per;
      int local = 0;
      for (int i = 0; i < per; ++i) local += e0 + i < f.E ? __popc(tmask[e0 + i]) : 0;
      int incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      int run = incl - local;
      for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < f.E) {
          route.offsets[e] = run;
          start[e] = run;
          run += __popc(tmask[e]);
        }
      }
      if (lane == 63) route.offsets[f.E] = incl;
      __builtin_amdgcn_wave_barrier();
      for (int a = lane; a < f.T * f.k; a += 64) {
        int e = route.ids[a];
        e = (unsigned)e < (unsigned)f.E ? e : f.E - 1;
        const int t = a / f.k;
        const int p = start[e] + __popc(tmask[e] & ((1u << t) - 1u));
        route.sorted[p] = a;
        route.pos[a] = p;
      }
      __builtin_amdgcn_wave_barrier();
    }
    const int n_all = n_routed + (f.Is > 0 ? 1 : 0);
    sb_begin = list_begin_idx == kPlanStart ? 0 : (list_begin_idx == kPlanRoutedBlocks ? n_routed : n_all);
    sb_end = list_end_idx == kPlanRoutedBlocks ? n_routed : n_all;
  } else {
    sb_begin = list_begin_idx == kPlanStart ? 0 : f.plan[list_begin_idx];
    sb_end = f.plan[list_end_idx];
  }
  const int wide = PHASE == 1 ? (f.I > f.Is ? f.I : f.Is) : f.H;
  const int cols_per_item = PHASE == 1 ? (SPLIT ? 8 : 16) : 32;
  const int n_slabs = (wide + cols_per_item - 1) / cols_per_item;
  const int total = (sb_end - sb_begin) * n_slabs;

  for (int item = gw; item < total; item += nw) {
    const int sb = sb_begin + item / n_slabs;
    const int slab = item % n_slabs;
    int g, r0, base, nrows;
    uint32_t mk = 0u;
    if (routed) {
      const int entry = glist[sb];
      g = entry & 2047;
      r0 = 0;
      if (g < f.E) {
        mk = (uint32_t)entry >> 11;
        nrows = __popc(mk);
        // first dispatched row: the rows of the experts listed before it
        int cnt = 0;
        for (int j = lane; j < sb; j += 64) cnt += __popc((uint32_t)glist[j] >> 11);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
        base = cnt;
      } else {
        base = 0;
        nrows = f.T;
      }
    } else if (self_plan) {
      g = glist[sb];
      r0 = 0;
      base = g < f.E ? f.offsets[g] : 0;
      nrows = g < f.E ? f.offsets[g + 1] - base : f.T;
    } else {
      g = f.sb_group[sb];
      r0 = f.sb_row0[sb];
      base = f.sb_base[sb];
      nrows = f.sb_nrows[sb];
    }
    stream_item<PHASE, FP8, SPLIT>(f, g, r0, base, nrows, self_plan ? nullptr : f.sb_tok + sb * kStreamBM, slab,
                                   lane, stage + wave * STAGE_BYTES, mk);
  }
}

// Router for T <= 16 (a GEMV bound by reading W_r): workgroup (s, y) of RW
// waves covers 16 router rows (the shared-gate row counted as row E) over K
// chunk y; its waves take consecutive sub-chunks, their partial 16x16 blocks
// are added through LDS in wave order, and the workgroup writes partial
// logits [y][T][N], which the top-k kernel adds in chunk order.
constexpr int RW = 8;

__global__ __launch_bounds__(RW * 64) void router_stream_kernel(const bf16* __restrict__ x,
                                                                const bf16* __restrict__ wr,
                                                                const bf16* __restrict__ wsg,
                                                                float* __restrict__ logits, int T, int H, int E,
                                                                int N, int kchunk, int32_t* zero_word) {
  // a word the next kernel in the chain needs at zero (or null)
  if (zero_word && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *zero_word = 0;
  __shared__ f32x4 part[RW][64];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int slab = blockIdx.x;
  const int m = lane & 15, kq = (lane >> 4) * 8;
  // workgroup blockIdx.y covers K values [y * RW * kchunk, +RW * kchunk) and
  // writes its own partial logits
  const int kbeg = (blockIdx.y * RW + w) * kchunk;
  const int kend = kbeg + kchunk < H ? kbeg + kchunk : H;
  logits += (int64_t)blockIdx.y * T * N;
  f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
  if (kbeg < kend) {
    const bf16* a_row = m < T ? x + (int64_t)m * H : nullptr;
    int n = slab * 16 + m;
    n = n < N ? n : N - 1;
    const bf16* b_row[1] = {n < E ? wr + (int64_t)n * H : wsg};
    stream_dot<1>(a_row, b_row, kbeg, kend, kq, acc);
  }
  part[w][lane] = acc[0];
  __syncthreads();
  if (w == 0) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int i = 1; i < RW; ++i) t += part[i][lane];
    const int col = slab * 16 + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * (lane >> 4) + i;
      if (tok < T && col < N) logits[(int64_t)tok * N + col] = t[i];
    }
  }
}

int stream_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    g = cus * 8;  // 8 workgroups (32 waves) per CU
  }
  return g;
}

}  // namespace

int router_stream_split(int H) {
  // about 128 K values per wave, so that each wave's loads fit in one batch
  // and the few (E + 1) / 16 row slabs still spread over many CUs
  const int ks = (H + RW * 128 - 1) / (RW * 128);
  return ks < 1 ? 1 : (ks > 16 ? 16 : ks);
}

hipError_t launch_router_stream(const void* x, const void* w_router, const void* w_sg, float* logits, int T, int H,
                                int E, int nsplit, hipStream_t s, int32_t* zero_word) {
  const int N = E + (w_sg ? 1 : 0);
  int kchunk = (H + RW * nsplit - 1) / (RW * nsplit);
  kchunk = (kchunk + KSTEP - 1) / KSTEP * KSTEP;
  router_stream_kernel<<<dim3((N + 15) / 16, nsplit), RW * 64, 0, s>>>(reinterpret_cast<const bf16*>(x),
                                                         reinterpret_cast<const bf16*>(w_router),
                                                         reinterpret_cast<const bf16*>(w_sg), logits, T, H, E, N,
                                                         kchunk, zero_word);
  return hipGetLastError();
}

hipError_t launch_ffn_stream(const FfnArgs& a, int phase, hipStream_t s, bool self_plan, const SmallRoute* route) {
  const int grid = stream_grid();
  const int blk = WAVES * 64;
  int sp = self_plan ? 1 : 0;
  // a batch of at most kStreamMaxRows tokens streams every group: split items
  const bool split = a.T <= kStreamMaxRows;
  SmallRoute r{nullptr, nullptr, nullptr, nullptr};
  if (route) {
    // the dispatch from the ids: bf16 gate/up of a small batch listing its own groups
    if (phase != 1 || a.fp8 || !self_plan || a.T > kSmallBatch || a.E > kMaxExperts || !route->ids ||
        !route->offsets || !route->sorted || !route->pos)
      return hipErrorInvalidValue;
    r = *route;
    sp = 2;
  }
  if (a.fp8) {
    if (phase == 1) stream_kernel<1, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanRoutedBlocks, sp, r);
    else stream_kernel<2, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanRoutedBlocks, sp, r);
    if (a.Is > 0) {
      if (phase == 1 && split)
        stream_kernel<1, false, true><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp, r);
      else if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp, r);
      else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp, r);
    }
  } else {
    if (phase == 1 && split) stream_kernel<1, false, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp, r);
    else if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp, r);
    else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp, r);
  }
  return hipGetLastError();
}

}  // namespace moe
