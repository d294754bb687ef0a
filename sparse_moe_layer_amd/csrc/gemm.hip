// Grouped expert GEMM on CDNA4 MFMA (v_mfma_f32_32x32x16_bf16), LDS-tiled.
//
// One kernel template covers the three dense contractions of the layer
// (Qwen3.8-Flash-Next study, "MoE: 512 experts behind a width-640
// intermediate": Router [T, E] and the grouped expert GEMMs of eq. expert(x)):
//   ROUTER : logits[t, n] = x_t . W_r[n]  (n < E) and x_t . w_sg (n == E), fp32 out
//   GATEUP : h[r, j] = SiLU(x_t . W_gate[e][j]) * (x_t . W_up[e][j]),  t = sorted[r]/k
//   DOWN   : y[r, n] = h[r] . W_down[e][n]
// Every operand is K-contiguous (x rows, weight rows, h rows), so both MFMA
// fragments are 16-byte LDS reads along K.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (4 waves in 2 x 2,
// 64 x 64 per wave = 2 x 2 MFMA 32x32 blocks), K step 64, two LDS buffers
// (64 KB).  The gate/up tile interleaves 32 gate rows and 32 up rows per wave
// so SiLU(g)*u is formed in registers.  Work is a device-built list of
// (group, first row) m-tiles; the grid is persistent and walks
// m-tile x n-tile indices, so no host sync is needed to size it.
// fp8 routed weights are decoded (OCP e4m3fn x fp32 block scale -> bf16) on
// their way into LDS.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BM = kGemmBM;
constexpr int BN = 128;
constexpr int BK = 64;
// K step of the bf16 expert tiles.  32 (half the LDS, three workgroups per
// CU) measured 19% slower on 4096 x 2560 gate/up than 64 with two.
constexpr int kBf16FfnBK = 64;
constexpr int NT = 256;

enum { M_ROUTER = 0, M_GATEUP = 1, M_DOWN = 2 };

struct RouterArgs {
  const bf16* x;
  const bf16* wr;
  const bf16* wsg;  // may be null
  float* logits;    // [nsplit][T, N] partial logits (K split into nsplit chunks)
  int T, H, E, N;
  int nsplit, kchunk;
};

// Element offset of the 16-byte chunk `c` of tile row `r`.  Rows are 128 B;
// gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a time over 64 banks
// (256 B), i.e. two rows per bank sweep, so the chunk is XOR-ed with
// (r >> 1) & 7: the 16 rows a half-wave reads land on 16 distinct 16-byte
// bank groups.
// With a 32-wide K step rows are 64 B and the chunk is XOR-ed with
// (r >> 2) & 3 for the same effect.
template <int BKT>
__device__ __forceinline__ int lds_off(int r, int c) {
  return BKT == 64 ? r * 64 + ((c ^ ((r >> 1) & 7)) << 3) : r * 32 + ((c ^ ((r >> 2) & 3)) << 3);
}

// USE tells apart launches of the same code for different callers in traces
// (0: the layer; 1: the gated residual's read projection).  BKT is the K step:
// 64 (two 64 KB LDS buffers, two workgroups per CU) or 32 (bf16 only: 32 KB,
// three workgroups per CU).
template <int MODE, bool FP8, int USE = 0, int BKT = 64>
__global__ __launch_bounds__(NT, BKT == 32 ? 3 : 2) void gemm_kernel(FfnArgs f, RouterArgs ra, int n_tiles_n,
                                                     int list_begin_idx, int list_end_idx) {
  static_assert(!FP8 || BKT == 64, "fp8 tiles use the 64-wide K step");
  constexpr int CPR = BKT / 8;     // 16-byte chunks per LDS row
  constexpr int RSTEP = NT / CPR;  // rows covered by one pass of the workgroup
  constexpr int NPASS = BM / RSTEP;
  __shared__ __attribute__((aligned(16))) bf16 sA[2 * BM * BKT];
  __shared__ __attribute__((aligned(16))) bf16 sB[2 * BN * BKT];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int mt_begin, mt_end;
  if (MODE == M_ROUTER) {
    mt_begin = 0;
    mt_end = (ra.T + BM - 1) / BM;
  } else {
    // plan ints: [0] first-list m-tiles, [2] its routed ones (shared ones
    // follow), [4] / [5] the second list
    mt_begin = list_begin_idx == kPlanStart ? 0 : f.plan[list_begin_idx];
    mt_end = f.plan[list_end_idx];
  }
  const int nsplit = MODE == M_ROUTER ? ra.nsplit : 1;
  const int total = (mt_end - mt_begin) * n_tiles_n * nsplit;

  // Workgroup i runs on XCD i % 8: deal consecutive tile indices to one XCD
  // (n-tiles and K chunks of an m-tile vary fastest), so the gathered A rows
  // of an m-tile are fetched into one XCD's L2 and reused from there.
  const int G8 = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const bool remap = (gridDim.x & 7) == 0;
  for (int it = 0;; ++it) {
    const int tile = remap ? it * gridDim.x + xcd * G8 + slot : it * gridDim.x + blockIdx.x;
    if (tile >= total) break;
    const int mt = mt_begin + tile / (n_tiles_n * nsplit);
    const int rem = tile % (n_tiles_n * nsplit);
    const int nt = rem % n_tiles_n;
    const int kc = rem / n_tiles_n;  // K chunk (router split-K)

    // ---------------- resolve the group of this m-tile ----------------
    int g = 0, base = 0, r0, nrows, K, Ncols;
    int kbeg = 0;
    if (MODE == M_ROUTER) {
      r0 = mt * BM;
      nrows = ra.T - r0;
      kbeg = kc * ra.kchunk;
      K = kbeg + ra.kchunk < ra.H ? kbeg + ra.kchunk : ra.H;  // end of this K chunk
      Ncols = ra.N;
    } else {
      g = f.mt_group[mt];
      r0 = f.mt_row0[mt];
      const bool shared = g >= f.E;
      if (!shared) {
        base = f.offsets[g];
        nrows = f.offsets[g + 1] - base - r0;
      } else {
        nrows = f.T - r0;
      }
      if (MODE == M_GATEUP) {
        K = f.H;
        Ncols = shared ? f.Is : f.I;
      } else {
        K = shared ? f.Is : f.I;
        Ncols = f.H;
      }
    }
    nrows = nrows < BM ? nrows : BM;
    const bool shared = (MODE != M_ROUTER) && g >= f.E;
    const bool fp8_tile = FP8 && !shared;
    // n-tile coverage: GATEUP covers 64 hidden columns per tile, others 128.
    const int ncov = (MODE == M_GATEUP) ? 64 : BN;
    if (nt * ncov >= Ncols) continue;  // uniform across the block

    // ---------------- per-thread operand row pointers ----------------
    const bf16* a_ptr[4];
    bool a_in[4];  // the row is one of the group's (rows past it are never stored)
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
      int r = tid / CPR + RSTEP * i;
      a_in[i] = r < nrows;
      r = r < nrows ? r : nrows - 1;  // clamp: rows past the group are computed, never stored
      const int gr = base + r0 + r;
      if (MODE == M_ROUTER) {
        a_ptr[i] = ra.x + (int64_t)gr * ra.H;
      } else if (MODE == M_GATEUP) {
        int tok = shared ? gr : f.sorted[gr] / f.k;
        tok = (unsigned)tok < (unsigned)f.T ? tok : f.T - 1;  // also clamps a negative index
        a_ptr[i] = reinterpret_cast<const bf16*>(f.x) + (int64_t)tok * f.H;
      } else {
        a_ptr[i] = shared ? reinterpret_cast<const bf16*>(f.h_sh) + (int64_t)gr * f.Is
                          : reinterpret_cast<const bf16*>(f.h) + (int64_t)gr * f.I;
      }
    }
    // B rows: bf16 layout uses rows tid/CPR + RSTEP*i, chunk tid%CPR (NPASS
    // chunks); fp8 layout uses rows (tid>>2)+64i, 16-code chunk tid&3 (2 chunks).
    const void* b_ptr[4];
    const float* s_ptr[4];
    const int nb = fp8_tile ? 2 : NPASS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= nb) { b_ptr[i] = nullptr; s_ptr[i] = nullptr; continue; }
      const int n = fp8_tile ? (tid >> 2) + 64 * i : tid / CPR + RSTEP * i;
      int col;  // matrix row of the weight (output column)
      bool up = false;
      if (MODE == M_GATEUP) {
        const int within = n & 63;
        up = within >= 32;
        col = nt * 64 + (n >> 6) * 32 + (within & 31);
      } else {
        col = nt * BN + n;
      }
      col = col < Ncols ? col : Ncols - 1;
      if (MODE == M_ROUTER) {
        b_ptr[i] = col < ra.E ? ra.wr + (int64_t)col * ra.H : ra.wsg;
        s_ptr[i] = nullptr;
      } else if (MODE == M_GATEUP) {
        if (shared) {
          b_ptr[i] = reinterpret_cast<const bf16*>(up ? f.shu : f.shg) + (int64_t)col * f.H;
          s_ptr[i] = nullptr;
        } else if (fp8_tile) {
          b_ptr[i] = reinterpret_cast<const uint8_t*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg) +
                     (int64_t)col * f.H;
          const int kb = f.H / 128;
          s_ptr[i] = (up ? f.scu : f.scg) + (int64_t)g * (f.I / 128) * kb + (col / 128) * kb;
        } else {
          b_ptr[i] = reinterpret_cast<const bf16*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg) +
                     (int64_t)col * f.H;
          s_ptr[i] = nullptr;
        }
      } else {
        if (shared) {
          b_ptr[i] = reinterpret_cast<const bf16*>(f.shd) + (int64_t)col * f.Is;
          s_ptr[i] = nullptr;
        } else if (fp8_tile) {
          b_ptr[i] = reinterpret_cast<const uint8_t*>(f.wd) + (int64_t)g * f.sd + (int64_t)col * f.I;
          const int kb = f.I / 128;
          s_ptr[i] = f.scd + (int64_t)g * (f.H / 128) * kb + (col / 128) * kb;
        } else {
          b_ptr[i] = reinterpret_cast<const bf16*>(f.wd) + (int64_t)g * f.sd + (int64_t)col * f.I;
          s_ptr[i] = nullptr;
        }
      }
    }

    // ---------------- main loop ----------------
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // fp8 weights: two register stages, the loads of K step kt+2 are issued
    // while step kt computes from LDS and step kt+1's registers are decoded
    // into LDS, so two steps' loads are in flight per workgroup (past the last
    // step the loads repeat it, never stored).  bf16: one register stage.
    u32x4 ra_reg[2][4], rb_reg[2][4];
    float rs_reg[2][2];
    const int kcol = tid % CPR;
    const int nk = (K - kbeg + BKT - 1) / BKT;

    auto gload = [&](int kt, int rb) {
      kt = kt < nk ? kt : nk - 1;
      const int k0 = kbeg + kt * BKT;
      // loads are unconditional (address clamped into the row, value zeroed
      // past K) so that no branch splits the load stream; skipping the padded
      // activation rows here, as the bf16 path does, measured no faster
      const int kk = k0 + kcol * 8;
      const bool kin = kk < K;
      const int kc = kin ? kk : K - 8;
#pragma unroll
      for (int i = 0; i < NPASS; ++i) {
        const u32x4 v = ld16(a_ptr[i] + kc);
        ra_reg[rb][i] = kin ? v : u32x4{0, 0, 0, 0};
      }
      if (fp8_tile) {
        const int kk = k0 + (tid & 3) * 16;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          rb_reg[rb][i] = ld16(reinterpret_cast<const uint8_t*>(b_ptr[i]) + kk);
          rs_reg[rb][i] = s_ptr[i][k0 / 128];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = ld16(reinterpret_cast<const bf16*>(b_ptr[i]) + kc);
          rb_reg[rb][i] = kin ? v : u32x4{0, 0, 0, 0};
        }
      }
    };
    auto lstore = [&](int buf, int rb) {
      bf16* a = sA + buf * BM * BKT;
      bf16* b = sB + buf * BN * BKT;
#pragma unroll
      for (int i = 0; i < NPASS; ++i) {
        const int r = tid / CPR + RSTEP * i;
        *reinterpret_cast<u32x4*>(a + lds_off<BKT>(r, kcol)) = ra_reg[rb][i];
      }
      if (fp8_tile) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = (tid >> 2) + 64 * i;
          const int c = (tid & 3) * 2;
          u32x2 lo = {rb_reg[rb][i][0], rb_reg[rb][i][1]};
          u32x2 hi = {rb_reg[rb][i][2], rb_reg[rb][i][3]};
          *reinterpret_cast<u32x4*>(b + lds_off<BKT>(r, c)) = fp8x8_to_bf16x8(lo, rs_reg[rb][i]);
          *reinterpret_cast<u32x4*>(b + lds_off<BKT>(r, c + 1)) = fp8x8_to_bf16x8(hi, rs_reg[rb][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
          const int r = tid / CPR + RSTEP * i;
          *reinterpret_cast<u32x4*>(b + lds_off<BKT>(r, kcol)) = rb_reg[rb][i];
        }
      }
    };
    auto compute = [&](int buf) {
      const bf16* a = sA + buf * BM * BKT;
      const bf16* b = sB + buf * BN * BKT;
#pragma unroll
      for (int ks = 0; ks < BKT / 16; ++ks) {
        const int c = ks * 2 + (lane >> 5);
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + (lane & 31);
          af[i] = *reinterpret_cast<const bf16x8*>(a + lds_off<BKT>(r, c));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wn * 64 + j * 32 + (lane & 31);
          bfr[j] = *reinterpret_cast<const bf16x8*>(b + lds_off<BKT>(r, c));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    };
    // step kt computes from LDS buffer kt%2 == P, refills register stage P
    // with step kt+2 and moves register stage 1-P (step kt+1) into LDS.
    auto step = [&](int kt, auto P) {
      constexpr int p = decltype(P)::value;
      gload(kt + 2, p);
      compute(p);
      if (kt + 1 < nk) lstore(1 - p, 1 - p);
      __syncthreads();
    };

    if constexpr (FP8) {
      gload(0, 0);
      gload(1, 1);
      lstore(0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
      }
    } else {
      // bf16 weights: one register stage with loads guarded per lane (both
      // measured faster for ~100-row groups than two stages or clamped loads).
      // Activation rows past the group are not loaded at all: in a 128-row
      // tile over a ~80-row expert they would be a third of the A loads.
      auto gload1 = [&](int kt) {
        const int k0 = kbeg + kt * BKT;
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
          const int kk = k0 + kcol * 8;
          ra_reg[0][i] = (kk < K && a_in[i]) ? ld16(a_ptr[i] + kk) : u32x4{0, 0, 0, 0};
        }
        // expert weights are non-temporal: a 128-row m-tile covers a
        // Flash-Next prefill group whole, so each weight line is read once
        // (gate/up 0.770 -> 0.741 ms); the router's weights serve every
        // m-tile and stay cached
#pragma unroll
        for (int i = 0; i < NPASS; ++i) {
          const int kk = k0 + kcol * 8;
          const bf16* bp = reinterpret_cast<const bf16*>(b_ptr[i]) + kk;
          u32x4 v = u32x4{0, 0, 0, 0};
          if (kk < K) {
            if constexpr (MODE == M_ROUTER) v = ld16(bp);
            else v = ld16_nt(bp);
          }
          rb_reg[0][i] = v;
        }
      };
      gload1(0);
      lstore(0, 0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload1(kt + 1);
        compute(buf);
        if (kt + 1 < nk) lstore(buf ^ 1, 0);
        __syncthreads();
      }
    }

    // ---------------- epilogue ----------------
    // C fragment: lane holds column (lane & 31), rows 8*(v/4) + 4*(lane/32) + v%4.
    if constexpr (MODE != M_ROUTER && BKT == 64) {
      // Through LDS (the K loop ended with a barrier, so sA is free): the
      // tile goes into sA as bf16 (gate/up: SiLU(g)*u), then every thread
      // stores whole 16-byte row chunks (bf16 rows are multiples of 8
      // elements).  Chunk c of row r sits at c ^ (4 * ((r >> 2) & 1)), so the
      // two half-waves' rows (4 apart) write different banks.
      constexpr int CC = MODE == M_GATEUP ? 64 : BN;  // output columns of the tile
      constexpr int CPRO = CC / 8;                   // 16-byte chunks per row
      static_assert(BM * CC <= 2 * BM * BKT, "the C tile fits the A buffers");
      auto cpos = [](int r, int col) { return r * CC + (((col >> 3) ^ (((r >> 2) & 1) << 2)) << 3) + (col & 7); };
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (MODE == M_GATEUP) {
            sA[cpos(rl, wn * 32 + (lane & 31))] = f2bf(silu(acc[i][0][v]) * acc[i][1][v]);
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) sA[cpos(rl, wn * 64 + j * 32 + (lane & 31))] = f2bf(acc[i][j][v]);
          }
        }
      }
      __syncthreads();
      bf16* obase;
      int ld;
      if (MODE == M_GATEUP) {
        obase = shared ? reinterpret_cast<bf16*>(f.h_sh) : reinterpret_cast<bf16*>(f.h);
        ld = shared ? f.Is : f.I;
      } else {
        obase = shared ? reinterpret_cast<bf16*>(f.y_sh) : reinterpret_cast<bf16*>(f.y);
        ld = f.H;
      }
      // non-temporal: h and y are read back only by the next launch (Flash-Next prefill
      // 1.30 -> 1.29 ms per step; in the 256-row tiles the same hint measured no gain)
      for (int q = tid; q < BM * CPRO; q += NT) {
        const int r = q / CPRO, c = q % CPRO;
        const int col = nt * CC + c * 8;
        if (r < nrows && col < Ncols) st16_nt(obase + (int64_t)(base + r0 + r) * ld + col, ld16(sA + cpos(r, c * 8)));
      }
      __syncthreads();  // sA is read out before the next tile refills it
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rl = wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          if (rl >= nrows) continue;
          const int64_t gr = base + r0 + rl;
          if (MODE == M_GATEUP) {
            const int col = nt * 64 + wn * 32 + (lane & 31);
            if (col < Ncols) {
              const float hv = silu(acc[i][0][v]) * acc[i][1][v];
              bf16* dst = shared ? reinterpret_cast<bf16*>(f.h_sh) + gr * f.Is
                                 : reinterpret_cast<bf16*>(f.h) + gr * f.I;
              dst[col] = f2bf(hv);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int col = nt * BN + wn * 64 + j * 32 + (lane & 31);
              if (col >= Ncols) continue;
              if (MODE == M_ROUTER) {
                ra.logits[((int64_t)kc * ra.T + gr) * ra.N + col] = acc[i][j][v];
              } else {
                bf16* dst = shared ? reinterpret_cast<bf16*>(f.y_sh) : reinterpret_cast<bf16*>(f.y);
                dst[gr * f.H + col] = f2bf(acc[i][j][v]);
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Work planning: per group (routed expert or the shared one) decide the path
// and emit (group, first row) entries for GEMM m-tiles and streaming m-blocks.
// Layout of plan ints:
//   [0] m-tiles of the first list  [1] stream m-blocks total
//   [2] first-list m-tiles of routed groups (the shared group's tiles follow)
//   [3] stream m-blocks of routed groups
//   [4], [5] the second m-tile list [plan[4], plan[5]) (256-row tiling:
//        groups' last m-tiles of at most 128 rows); [6], [7] unused
//   [kPlanHeader..]  mt_group[max_mt], mt_row0[max_mt], sb_group[max_sb],
//        sb_row0[max_sb], sb_base[max_sb], sb_nrows[max_sb], sb_tok[max_sb][kStreamBM]
// ---------------------------------------------------------------------------
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  // blockDim.x == 1024 (16 waves)
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int s = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(s, o, 64);
    if (lane >= o) s += t;
  }
  if (lane == 63) tmp[w] = s;
  __syncthreads();
  if (w == 0) {
    int t = lane < 16 ? tmp[lane] : 0;
    int u = t;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int q = __shfl_up(u, o, 64);
      if (lane >= o) u += q;
    }
    if (lane < 16) tmp[16 + lane] = u - t;
    if (lane == 15) *total = u;
  }
  __syncthreads();
  const int r = s - v + tmp[16 + w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* offsets, const int32_t* sorted, int T, int E,
                                                    int k, int has_shared, uint32_t flags, int bm, int stream_rows,
                                                    int32_t* plan, int max_mt, int max_sb) {
  __shared__ int tmp[32];
  __shared__ int tot;
  // the fused kernels' claim counters start at zero
  for (int i = threadIdx.x; i < kPlanHeader - kPlanCounters; i += blockDim.x) plan[kPlanCounters + i] = 0;
  int32_t* mt_group = plan + kPlanHeader;
  int32_t* mt_row0 = mt_group + max_mt;
  int32_t* sb_group = mt_row0 + max_mt;
  int32_t* sb_row0 = sb_group + max_sb;
  int32_t* sb_base = sb_row0 + max_sb;
  int32_t* sb_nrows = sb_base + max_sb;
  int32_t* sb_tok = sb_nrows + max_sb;
  const int G = E + (has_shared ? 1 : 0);
  int carry_mt = 0, carry_sb = 0;
  for (int g0 = 0; g0 < G; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int n = 0;
    if (g < E) n = offsets[g + 1] - offsets[g];
    else if (g < G) n = T;
    bool gemm = false;
    if (n > 0) {
      if (flags & 1u) gemm = true;            // force GEMM
      else if (flags & 2u) gemm = false;      // force streaming
      else gemm = n > stream_rows;
    }
    const int cm = gemm ? (n + bm - 1) / bm : 0;
    const int cs = (n > 0 && !gemm) ? (n + kStreamBM - 1) / kStreamBM : 0;
    // routed groups first in each list, the shared group (g == E) last: since
    // g ascends with the scan order, this holds automatically.
    const int om = block_excl_scan(cm, tmp, &tot) + carry_mt;
    const int tm = tot;
    const int os = block_excl_scan(cs, tmp, &tot) + carry_sb;
    const int ts = tot;
    for (int i = 0; i < cm; ++i) { mt_group[om + i] = g; mt_row0[om + i] = i * bm; }
    const int gbase = g < E ? offsets[g] : 0;
    for (int i = 0; i < cs; ++i) {
      const int sb = os + i, r0 = i * kStreamBM;
      const int nr = n - r0 < kStreamBM ? n - r0 : kStreamBM;
      sb_group[sb] = g;
      sb_row0[sb] = r0;
      sb_base[sb] = gbase;
      sb_nrows[sb] = nr;
      for (int m = 0; m < kStreamBM; ++m) {
        int tok = 0;
        if (m < nr) {  // sorted is null for the down phase alone, which needs no tokens
          tok = g < E ? (sorted ? sorted[gbase + r0 + m] / k : 0) : r0 + m;
          tok = (unsigned)tok < (unsigned)T ? tok : T - 1;
        }
        sb_tok[sb * kStreamBM + m] = tok;
      }
    }
    if (has_shared && g == E) {
      plan[2] = om;  // routed gemm tiles precede the shared group's
      plan[3] = os;
    }
    carry_mt += tm;
    carry_sb += ts;
  }
  if (threadIdx.x == 0) {
    plan[0] = carry_mt;
    plan[1] = carry_sb;
    if (!has_shared) { plan[2] = carry_mt; plan[3] = carry_sb; }
  }
}

inline int max_mtiles(int64_t T, int64_t E, int64_t k, bool shared) {
  return (int)((T * k + kGemmBM - 1) / kGemmBM + E + (shared ? (T + kGemmBM - 1) / kGemmBM + 1 : 0));
}
inline int max_sblocks(int64_t T, int64_t E, int64_t k, bool shared) {
  return (int)((T * k + kStreamBM - 1) / kStreamBM + E + (shared ? (T + kStreamBM - 1) / kStreamBM + 1 : 0));
}

int num_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

}  // namespace

size_t ffn_plan_ints(int64_t T, int64_t E, int64_t k, bool shared) {
  return kPlanHeader + 2 * (size_t)max_mtiles(T, E, k, shared) +
         (4 + kStreamBM) * (size_t)max_sblocks(T, E, k, shared);
}

void ffn_bind_plan(FfnArgs& a, int32_t* plan) {
  const bool sh = a.Is > 0;
  const int mm = max_mtiles(a.T, a.E, a.k, sh), ms = max_sblocks(a.T, a.E, a.k, sh);
  a.plan = plan;
  a.mt_group = plan + kPlanHeader;
  a.mt_row0 = a.mt_group + mm;
  a.sb_group = a.mt_row0 + mm;
  a.sb_row0 = a.sb_group + ms;
  a.sb_base = a.sb_row0 + ms;
  a.sb_nrows = a.sb_base + ms;
  a.sb_tok = a.sb_nrows + ms;
}

hipError_t launch_ffn_plan(const int32_t* offsets, const int32_t* sorted, int T, int E, int k, int has_shared,
                           uint32_t flags, int bm, int stream_rows, int32_t* plan, hipStream_t s) {
  // list capacity is sized for the smallest tile height (kGemmBM <= bm)
  const int mm = max_mtiles(T, E, k, has_shared), ms = max_sblocks(T, E, k, has_shared);
  plan_kernel<<<1, 1024, 0, s>>>(offsets, sorted, T, E, k, has_shared, flags, bm, stream_rows, plan, mm, ms);
  return hipGetLastError();
}

int router_gemm_split(int T, int H, int E, int max_split) {
  // as many (m, n, K-chunk) tiles as fit in one round of resident workgroups
  // (two per CU): a split that spills a few tiles into a second round
  // doubles the kernel's time.  Up to max_split chunks, a split whose rounds
  // cost less in K steps may take more than one round: the 8192-token
  // router's 320 tiles run as 960 thirds in two rounds of 512 (router and
  // top-k stage 0.208 -> 0.170 ms).  Chunks are whole 64-wide K steps.
  int tiles = ((T + BM - 1) / BM) * ((E + 1 + BN - 1) / BN);
  tiles = tiles < 1 ? 1 : tiles;  // an empty batch still sizes one split
  const int slots = 2 * num_cus();
  int ns = slots / tiles;
  const int maxs = H / (4 * BK) > 0 ? H / (4 * BK) : 1;
  ns = ns < 1 ? 1 : (ns > maxs ? maxs : ns);
  // rounds / ns is the time in units of one whole-K tile; keep the
  // one-round split unless a larger one is strictly cheaper
  auto cost = [&](int n) { return (double)((tiles * n + slots - 1) / slots) / n; };
  const int n1 = ns;
  for (int n = n1 + 1; n <= max_split && n <= maxs; ++n)
    if (cost(n) < cost(ns)) ns = n;
  int kchunk = (H + ns - 1) / ns;
  kchunk = (kchunk + BK - 1) / BK * BK;
  return (H + kchunk - 1) / kchunk;
}

hipError_t launch_router_logits_bf16(const void* x, const void* w_router, const void* w_sg, float* logits,
                                     int T, int H, int E, int nsplit, hipStream_t s, bool gated_residual) {
  int kchunk = (H + nsplit - 1) / nsplit;
  kchunk = (kchunk + BK - 1) / BK * BK;
  RouterArgs ra{reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(w_router),
                reinterpret_cast<const bf16*>(w_sg), logits, T, H, E, E + (w_sg ? 1 : 0), nsplit, kchunk};
  const int ntn = (ra.N + BN - 1) / BN;
  const int tiles = ((T + BM - 1) / BM) * ntn * nsplit;
  const int grid = tiles < num_cus() * 2 ? (tiles + 7) / 8 * 8 : num_cus() * 2;
  FfnArgs none{};
  if (gated_residual)
    gemm_kernel<M_ROUTER, false, 1><<<grid, NT, 0, s>>>(none, ra, ntn, kPlanStart, kPlanTiles);
  else
    gemm_kernel<M_ROUTER, false><<<grid, NT, 0, s>>>(none, ra, ntn, kPlanStart, kPlanTiles);
  return hipGetLastError();
}

// Tiled MFMA phase of the expert FFN (phase 1: gate/up + SiLU*mul, 2: down).
hipError_t launch_ffn_gemm(const FfnArgs& a, int phase, hipStream_t s) {
  const bool sh = a.Is > 0;
  const int mm = max_mtiles(a.T, a.E, a.k, sh);
  const int wide = a.I > a.Is ? a.I : a.Is;
  const int ntn = phase == 1 ? (wide + 63) / 64 : (a.H + BN - 1) / BN;
  const int64_t tiles = (int64_t)mm * ntn;
  const int grid = (int)(tiles < num_cus() * 2 ? (tiles + 7) / 8 * 8 : num_cus() * 2);
  RouterArgs none{};
  if (a.fp8) {
    // routed tiles [0, plan[2]) decode fp8; the shared expert stays bf16
    if (phase == 1) gemm_kernel<M_GATEUP, true><<<grid, NT, 0, s>>>(a, none, ntn, kPlanStart, kPlanRoutedTiles);
    else gemm_kernel<M_DOWN, true><<<grid, NT, 0, s>>>(a, none, ntn, kPlanStart, kPlanRoutedTiles);
    if (sh) {
      if (phase == 1) gemm_kernel<M_GATEUP, false><<<grid, NT, 0, s>>>(a, none, ntn, kPlanRoutedTiles, kPlanTiles);
      else gemm_kernel<M_DOWN, false><<<grid, NT, 0, s>>>(a, none, ntn, kPlanRoutedTiles, kPlanTiles);
    }
  } else {
    constexpr int per_cu = kBf16FfnBK == 32 ? 3 : 2;
    const int g3 = (int)(tiles < num_cus() * per_cu ? (tiles + 7) / 8 * 8 : num_cus() * per_cu);
    if (phase == 1)
      gemm_kernel<M_GATEUP, false, 0, kBf16FfnBK><<<g3, NT, 0, s>>>(a, none, ntn, kPlanStart, kPlanTiles);
    else gemm_kernel<M_DOWN, false, 0, kBf16FfnBK><<<g3, NT, 0, s>>>(a, none, ntn, kPlanStart, kPlanTiles);
  }
  return hipGetLastError();
}

}  // namespace moe
