// Weight-streaming contractions for groups with few rows (decode, skew tails)
// and the split-K router for small batches.
//
// When an expert holds only a handful of tokens the expert GEMMs of
// eq. expert(x) (Qwen3.8-Flash-Next study, MoE section) are bound by reading
// its weights once from HBM.  Each wave owns one (16-row m-block, weight slab)
// item and streams the slab's weight rows once from HBM (every weight byte
// is used by exactly one wave) into v_mfma_f32_16x16x32_bf16 B fragments
// (lane = weight row l%16, 8 consecutive K values).  HBM wants long runs per
// row: a fragment-shaped load touches 16 rows x 64 B and runs at well under
// half the bandwidth of 512-byte runs, so bf16 weights are loaded in 512-byte
// runs (each 16-byte-per-lane load covers 2 rows x 512 B), one batch of 256 K
// values ahead in registers, and re-laid into MFMA fragments through a
// wave-private LDS stage (no barriers).
// fp8 codes stream the same way in 256-byte runs (4 rows per load) and are
// decoded with their block scale as fragments leave LDS.  The (at most 16)
// activation rows come from L2.
//   gate/up item: 16 hidden columns (16 gate rows + 16 up rows), SiLU*mul in registers
//   down item   : 32 output columns (2 blocks of 16 W_down rows)
//   router item : 16 router rows (the shared-gate row last) over one K chunk,
//                 fp32 partial logits, reduced in fixed order by the top-k kernel
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int WAVES = 4;
constexpr int U = 4;  // K steps per batch
constexpr int KSTEP = 32;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

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

// ---- LDS-staged bf16 streaming -------------------------------------------
// A batch holds SB = 256 K values (512 B) of NB*16 weight rows.  Rows 2i and
// 2i+1 of the batch sit in 1 KB at i * 1040 B (1 KB + 16 B pad); odd rows
// store 16-byte chunk c at position c ^ 8.  A half-wave reading 16 rows of
// one chunk then hits 16 different 16-byte bank groups of the 64-bank LDS.
constexpr int SB = 256;
constexpr int PAIR = 1040;

// acc[j] += A[16 rows, kbeg..kend) x W_j[16 rows, kbeg..kend)^T.  a_row: this
// lane's activation row (row lane%16) or null (zero row); wrow0[j]: row 0 of
// weight block j (rows ldw elements apart), of which nvalid[j] rows exist
// (rows past them re-read the last one; their outputs are never stored);
// lds: this wave's NB*8*PAIR-byte stage buffer.
// Per batch each lane loads 16 B of weights per row pair (lanes 0-31 the even
// row, 32-63 the odd row: 512 contiguous bytes per row and instruction) into
// registers one batch ahead, writes them to the wave's LDS stage, and reads
// MFMA fragments back.  The steady-state loop is branch-free; every load is
// unconditional (clamped addresses, values zeroed after loading).
// SPLIT (NB == 1): the 16-row block is two halves, rows 0-7 from wrow0[0]
// and rows 8-15 from wrow0[1], with nvalid[0] and nvalid[1] valid rows.
// DEPTH: batches of weights (and activations) loaded ahead of the one being
// computed (2 doubles the bytes each wave keeps in flight; it needs the
// registers of a second weight batch).  With DEPTH 2 every load is issued
// unconditionally, so the compiler's load counters stay exact (a load under
// a branch makes it wait for everything at the join): the loads of the two
// batches past the end read one cached 16-byte chunk and are never used.
template <int NB, bool SPLIT = false, int DEPTH = 1>
__device__ __forceinline__ void stream_dot_lds(const bf16* a_row, const bf16* a_any, const bf16* const* wrow0,
                                               const int* nvalid, int ldw, int kbeg, int kend, int lane, char* lds,
                                               f32x4* acc) {
  static_assert(!SPLIT || NB == 1, "a split block is the only block");
  static_assert(DEPTH == 1 || DEPTH == 2, "load depth");
  constexpr int NL = NB * 8;      // weight loads per batch
  constexpr int NA = SB / KSTEP;  // activation loads per batch
  const int kq = (lane >> 4) * 8;
  const int h = lane >> 5;        // row of the pair this lane loads
  const int c = lane & 31;        // its 16-byte chunk of the 512-byte run
  const int nbatch = (kend - kbeg + SB - 1) / SB;
  const bf16* arow = a_row ? a_row : a_any;
  u32x4 wb[DEPTH][NL];  // weights of the batches in flight
  u32x4 av[2][NA];      // activations, double-buffered
  auto load_w = [&](int x, int b) {
    int k = kbeg + b * SB + c * 8;
    k = k < kend ? k : kend - 8;  // past the end: any in-row chunk (its A is zero)
    const bool live = DEPTH == 1 || b < nbatch;  // a batch past the end reads element 0
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (SPLIT) {
          const int half = i >> 2, rh = (2 * i + h) & 7;  // rows 0-7: first half, 8-15: second
          const int r = rh < nvalid[half] ? rh : nvalid[half] - 1;
          wb[x][i] = ld16(wrow0[half] + (live ? (uint32_t)(r * ldw + k) : 0u));
        } else {
          const int r = 2 * i + h < nvalid[j] ? 2 * i + h : nvalid[j] - 1;
          wb[x][j * 8 + i] = ld16(wrow0[j] + (live ? (uint32_t)(r * ldw + k) : 0u));
        }
      }
  };
  auto load_a = [&](int x, int b) {
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const int kk = kbeg + b * SB + s * KSTEP + kq;
      av[x][s] = ld16(arow + (kk < kend ? kk : kend - 8));
    }
  };
  auto stage = [&](int x) {
#pragma unroll
    for (int q = 0; q < NL; ++q)
      *reinterpret_cast<u32x4*>(lds + q * PAIR + h * 512 + ((c ^ (h << 3)) << 4)) = wb[x][q];
  };
  auto compute = [&](int x, int b) {
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const int kk = kbeg + b * SB + s * KSTEP + kq;
      const u32x4 am = (a_row && kk < kend) ? av[x][s] : u32x4{0, 0, 0, 0};
      const int cc = s * 4 + (lane >> 4);
      const int n = lane & 15;
      const int hn = n & 1;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(lds + (j * 8 + (n >> 1)) * PAIR + hn * 512 +
                                                         ((cc ^ (hn << 3)) << 4));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(am), as_bf16x8(bv), acc[j], 0, 0, 0);
      }
    }
  };
  if constexpr (DEPTH == 2) {
    // batch b (buffers x = b % 2): stage its weights, refill the weight
    // buffer with batch b+2, run batch b's MFMAs, refill the activation
    // buffer with batch b+2; batches b+1 and b+2 stay in flight meanwhile
    auto step = [&](int x, int b) {
      stage(x);
      load_w(x, b + 2);
      compute(x, b);
      load_a(x, b + 2);
    };
    load_w(0, 0);
    load_a(0, 0);
    load_w(1, 1);
    load_a(1, 1);
    for (int b = 0;; b += 2) {
      step(0, b);
      if (b + 1 >= nbatch) break;
      step(1, b + 1);
      if (b + 2 >= nbatch) break;
    }
  } else {
    // batch b: stage its weights (loaded during the previous batch), start
    // batch b+1's loads, run batch b's MFMAs from LDS
    load_w(0, 0);
    load_a(0, 0);
    int b = 0;
    for (; b + 2 < nbatch; b += 2) {
      stage(0);
      load_w(0, b + 1);
      load_a(1, b + 1);
      compute(0, b);
      stage(0);
      load_w(0, b + 2);
      load_a(0, b + 2);
      compute(1, b + 1);
    }
    stage(0);
    if (b + 1 < nbatch) {
      load_w(0, b + 1);
      load_a(1, b + 1);
      compute(0, b);
      stage(0);
      compute(1, b + 1);
    } else {
      compute(0, b);
    }
  }
}

// ---- LDS-staged fp8 streaming ----------------------------------------------
// Same scheme for e4m3fn codes: a batch holds SB8 = 256 K values (256 B) of
// NB*16 weight rows; rows 2i and 2i+1 sit in 512 B at i * 528 B, odd rows
// store chunk c at c ^ 8.  Each 16-byte-per-lane load covers 4 rows x 256
// contiguous bytes.  Fragments are decoded when read from LDS: 8 codes times
// the row's 128 x 128 block scale (s_row[j]: this lane's fragment row's scale
// row, indexed by k / 128) to eight bf16.
constexpr int SB8 = 256;
constexpr int PAIR8 = 528;

template <int NB>
__device__ __forceinline__ void stream_dot_lds8(const bf16* a_row, const bf16* a_any, const uint8_t* const* wrow0,
                                                const int* nvalid, int ldw, const float* const* s_row, int kbeg,
                                                int kend, int lane, char* lds, f32x4* acc) {
  constexpr int NL = NB * 4;       // weight loads per batch (4 rows each)
  constexpr int NA = SB8 / KSTEP;  // activation loads per batch
  const int kq = (lane >> 4) * 8;
  const int q4 = lane >> 4;        // row of the quad this lane loads
  const int c = lane & 15;         // its 16-byte chunk of the 256-byte run
  const int nbatch = (kend - kbeg + SB8 - 1) / SB8;
  const bf16* arow = a_row ? a_row : a_any;
  u32x4 wb[NL];
  u32x4 av[2][NA];
  float sc[2][NB][2];  // block scales of this lane's fragment row, two 128-wide K blocks per batch
  auto load_w = [&](int b) {
    int k = kbeg + b * SB8 + c * 16;
    k = k < kend ? k : kend - 16;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + q4 < nvalid[j] ? 4 * i + q4 : nvalid[j] - 1;
        wb[j * 4 + i] = ld16(wrow0[j] + (uint32_t)(r * ldw + k));
      }
  };
  auto load_a = [&](int x, int b) {
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const int kk = kbeg + b * SB8 + s * KSTEP + kq;
      av[x][s] = ld16(arow + (kk < kend ? kk : kend - 8));
    }
    const int kb = (kbeg + b * SB8) / 128;
    const int kbl = (kend - 1) / 128;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      sc[x][j][0] = s_row[j][kb < kbl ? kb : kbl];
      sc[x][j][1] = s_row[j][kb + 1 < kbl ? kb + 1 : kbl];
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + q4;
        *reinterpret_cast<u32x4*>(lds + (j * 8 + (r >> 1)) * PAIR8 + (r & 1) * 256 + ((c ^ ((r & 1) << 3)) << 4)) =
            wb[j * 4 + i];
      }
  };
  auto compute = [&](int x, int b) {
    const int n = lane & 15;
    const int hn = n & 1;
#pragma unroll
    for (int s = 0; s < NA; ++s) {
      const int kk = kbeg + b * SB8 + s * KSTEP + kq;
      const u32x4 am = (a_row && kk < kend) ? av[x][s] : u32x4{0, 0, 0, 0};
      const int byte = s * KSTEP + kq;  // offset in the 256-byte row run
      const int cc = byte >> 4;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const u32x2 codes = *reinterpret_cast<const u32x2*>(lds + (j * 8 + (n >> 1)) * PAIR8 + hn * 256 +
                                                            ((cc ^ (hn << 3)) << 4) + (byte & 15));
        const u32x4 bv = fp8x8_to_bf16x8(codes, sc[x][j][s >= NA / 2 ? 1 : 0]);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(am), as_bf16x8(bv), acc[j], 0, 0, 0);
      }
    }
  };
  load_w(0);
  load_a(0, 0);
  int b = 0;
  for (; b + 2 < nbatch; b += 2) {
    stage();
    load_w(b + 1);
    load_a(1, b + 1);
    compute(0, b);
    stage();
    load_w(b + 2);
    load_a(0, b + 2);
    compute(1, b + 1);
  }
  stage();
  if (b + 1 < nbatch) {
    load_w(b + 1);
    load_a(1, b + 1);
    compute(0, b);
    stage();
    compute(1, b + 1);
  } else {
    compute(0, b);
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
template <int PHASE, bool FP8, bool SPLIT = false>
__global__ __launch_bounds__(WAVES * 64, 2) void stream_kernel(FfnArgs f, int list_begin_idx, int list_end_idx,
                                                               int self_plan) {
  static_assert(!SPLIT || (PHASE == 1 && !FP8), "split items are bf16 gate/up");
  constexpr int NB = SPLIT ? 1 : 2;
  constexpr int STAGE_BYTES = NB * 8 * (FP8 ? PAIR8 : PAIR);  // per wave
  __shared__ __attribute__((aligned(16))) char stage[WAVES * STAGE_BYTES];
  __shared__ int glist[kMaxExperts + 1];  // SELF_PLAN: touched groups
  __shared__ int wtot[WAVES];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int nw = gridDim.x * WAVES;
  int sb_begin, sb_end;
  if (self_plan) {
    // ordered compaction of the routed groups with rows, 64*WAVES at a time:
    // a wave's ballot gives each lane its rank, the waves' totals its offset
    int n_routed = 0;
    for (int g0 = 0; g0 < f.E; g0 += WAVES * 64) {
      const int g = g0 + threadIdx.x;
      const bool t = g < f.E && f.offsets[g + 1] > f.offsets[g];
      const uint64_t bal = __ballot(t);
      const int rank = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wtot[wave] = __popcll(bal);
      __syncthreads();
      int off = n_routed;
      for (int w = 0; w < wave; ++w) off += wtot[w];
      if (t) glist[off + rank] = g;
      for (int w = 0; w < WAVES; ++w) n_routed += wtot[w];
      __syncthreads();
    }
    if (threadIdx.x == 0) glist[n_routed] = f.E;  // the shared expert (read only when present)
    __syncthreads();
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
  const int m = lane & 15;         // A row / B column within a 16-block

  for (int item = gw; item < total; item += nw) {
    const int sb = sb_begin + item / n_slabs;
    const int slab = item % n_slabs;
    int g, r0, base, nrows;
    if (self_plan) {
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
    const bool shared = g >= f.E;
    const int K = PHASE == 1 ? f.H : (shared ? f.Is : f.I);
    const int Ncols = PHASE == 1 ? (shared ? f.Is : f.I) : f.H;
    const int c0 = slab * cols_per_item;
    if (c0 >= Ncols) continue;

    // A row of this lane (zero when past the group's rows)
    const bf16* a_row = nullptr;
    if (m < nrows) {
      const int gr = base + r0 + m;
      if (PHASE == 1) {
        int tok;
        if (!self_plan) tok = f.sb_tok[sb * kStreamBM + m];
        else tok = g < f.E ? f.sorted[gr] / f.k : m;
        tok = tok < f.T ? tok : f.T - 1;
        a_row = reinterpret_cast<const bf16*>(f.x) + (int64_t)tok * f.H;
      } else {
        a_row = shared ? reinterpret_cast<const bf16*>(f.h_sh) + (int64_t)gr * f.Is
                       : reinterpret_cast<const bf16*>(f.h) + (int64_t)gr * f.I;
      }
    }
    // fp8: this lane's fragment row's block-scale row, one per 16-column block
    const float* s_row[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      s_row[j] = nullptr;
      if (FP8) {
        int col = PHASE == 1 ? c0 + m : c0 + j * 16 + m;
        col = col < Ncols ? col : Ncols - 1;
        if (PHASE == 1) {
          const int kb = f.H / 128;
          s_row[j] = (j ? f.scu : f.scg) + (int64_t)g * (f.I / 128) * kb + (col / 128) * kb;
        } else {
          const int kb = f.I / 128;
          s_row[j] = f.scd + (int64_t)g * (f.H / 128) * kb + (col / 128) * kb;
        }
      }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FP8) {
      // (an fp8 launch covers the routed groups only; the shared expert's
      // bf16 weights go through the bf16 launch)
      // first row and valid-row count of each 16-row weight block, and this
      // lane's fragment row's scale row
      const uint8_t* w0[NB];
      int nv[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        int first = PHASE == 1 ? c0 : c0 + j * 16;
        first = first < Ncols ? first : Ncols - 1;
        nv[j] = Ncols - first;
        const uint8_t* mat = PHASE == 1
                                 ? reinterpret_cast<const uint8_t*>(j ? f.wu : f.wg) + (int64_t)g * (j ? f.su : f.sg)
                                 : reinterpret_cast<const uint8_t*>(f.wd) + (int64_t)g * f.sd;
        w0[j] = mat + (int64_t)first * K;
      }
      const bf16* a_any = reinterpret_cast<const bf16*>(PHASE == 1 ? f.x : f.h);
      stream_dot_lds8<NB>(a_row, a_any, w0, nv, K, s_row, 0, K, lane, stage + wave * STAGE_BYTES, acc);
    } else {
      // first row and valid-row count of each weight block (gate/up: of the
      // gate half and the up half of the one split block)
      constexpr int NW0 = SPLIT ? 2 : NB;
      const bf16* w0[NW0];
      int nv[NW0];
#pragma unroll
      for (int j = 0; j < NW0; ++j) {
        int first = PHASE == 1 ? c0 : c0 + j * 16;
        first = first < Ncols ? first : Ncols - 1;
        nv[j] = Ncols - first;
        const bf16* mat;
        if (PHASE == 1) {
          mat = shared ? reinterpret_cast<const bf16*>(j ? f.shu : f.shg)
                       : reinterpret_cast<const bf16*>(j ? f.wu : f.wg) + (int64_t)g * (j ? f.su : f.sg);
        } else {
          mat = shared ? reinterpret_cast<const bf16*>(f.shd) : reinterpret_cast<const bf16*>(f.wd) + (int64_t)g * f.sd;
        }
        w0[j] = mat + (int64_t)first * K;
      }
      const bf16* a_any = reinterpret_cast<const bf16*>(PHASE == 1 ? f.x : (shared ? f.h_sh : f.h));
      stream_dot_lds<NB, SPLIT, SPLIT ? 2 : 1>(a_row, a_any, w0, nv, K, 0, K, lane, stage + wave * STAGE_BYTES, acc);
    }

    // C fragment: lane holds column (lane & 15), rows 4*(lane>>4) + i.  A split
    // gate/up block has the up column of lane m (m < 8) in lane m + 8.
    float up_v[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) up_v[i] = __shfl_xor(acc[0][i], 8, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (row >= nrows) continue;
      const int64_t gr = base + r0 + row;
      if (PHASE == 1) {
        bf16* dst = shared ? reinterpret_cast<bf16*>(f.h_sh) + gr * f.Is : reinterpret_cast<bf16*>(f.h) + gr * f.I;
        if constexpr (SPLIT) {
          // lane column m: gate column c0 + m (m < 8), up column c0 + m - 8 (m >= 8)
          const int col = c0 + m;
          if (m < 8 && col < Ncols) dst[col] = f2bf(silu(acc[0][i]) * up_v[i]);
        } else {
          const int col = c0 + m;
          if (col < Ncols) dst[col] = f2bf(silu(acc[0][i]) * acc[1][i]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = c0 + j * 16 + m;
          if (col < Ncols) {
            bf16* dst = shared ? reinterpret_cast<bf16*>(f.y_sh) : reinterpret_cast<bf16*>(f.y);
            dst[gr * f.H + col] = f2bf(acc[j][i]);
          }
        }
      }
    }
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
                                                                int N, int kchunk) {
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
                                int E, int nsplit, hipStream_t s) {
  const int N = E + (w_sg ? 1 : 0);
  int kchunk = (H + RW * nsplit - 1) / (RW * nsplit);
  kchunk = (kchunk + KSTEP - 1) / KSTEP * KSTEP;
  router_stream_kernel<<<dim3((N + 15) / 16, nsplit), RW * 64, 0, s>>>(reinterpret_cast<const bf16*>(x),
                                                         reinterpret_cast<const bf16*>(w_router),
                                                         reinterpret_cast<const bf16*>(w_sg), logits, T, H, E, N,
                                                         kchunk);
  return hipGetLastError();
}

hipError_t launch_ffn_stream(const FfnArgs& a, int phase, hipStream_t s, bool self_plan) {
  const int grid = stream_grid();
  const int blk = WAVES * 64;
  const int sp = self_plan ? 1 : 0;
  // a batch of at most kStreamMaxRows tokens streams every group: split items
  const bool split = a.T <= kStreamMaxRows;
  if (a.fp8) {
    if (phase == 1) stream_kernel<1, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanRoutedBlocks, sp);
    else stream_kernel<2, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanRoutedBlocks, sp);
    if (a.Is > 0) {
      if (phase == 1 && split) stream_kernel<1, false, true><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp);
      else if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp);
      else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, kPlanRoutedBlocks, kPlanBlocks, sp);
    }
  } else {
    if (phase == 1 && split) stream_kernel<1, false, true><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp);
    else if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp);
    else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, kPlanStart, kPlanBlocks, sp);
  }
  return hipGetLastError();
}

}  // namespace moe
