// Big-tile grouped expert GEMM for compute-bound groups (many rows per
// expert), gfx950: the gate/up and down contractions of eq. expert(x) in the
// Qwen3.8-Flash-Next study's MoE section, on v_mfma_f32_32x32x16_bf16.
//
// Tile 256 x 256, K step 32, 512 threads = 8 waves (two per SIMD, so one
// wave's MFMAs cover the other's LDS waits), each wave 128 x 64 (4 x 2
// blocks of 32 x 32, 128 fp32 accumulators).  A wave owns M-blocks
// {wm, wm+2, wm+4, wm+6} (interleaved, so a partial tile of 64 or 128 rows
// keeps every wave busy) and N-blocks 2*wn, 2*wn+1.  For gate/up a wave's two
// N-blocks are 32 gate rows and the 32 up rows of the same hidden columns, so
// SiLU(g)*u is formed in registers.
//
// Operands move HBM/L2 -> LDS with gfx950's direct loads (global_load_lds
// 16 bytes per lane; no VGPR staging) into two statically separate stage
// buffers; waits are explicit s_waitcnt vmcnt + s_barrier.  The LDS image of
// a 64-wide K slice is [row][8 chunks of 16 B] with chunk c of row r stored
// at position c ^ ((r >> 1) & 7) (a half-wave's 16-byte reads cover 16 rows;
// 64 banks hold two 128-byte rows, so this spreads them over all banks); a
// lane's direct load picks the global chunk that belongs at its LDS
// position, so rows stay fully coalesced.
//
// Work: (group, 256-row m-tile) entries from the device plan; tiles are
// ordered in supertiles of 8 m-tiles x all n-tiles and dealt to the
// persistent grid so that 32 consecutive tiles land on one XCD (workgroup i
// runs on XCD i mod 8): they share 8 A slices and 4 weight slices per K step
// in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BM = kGemmBigBM;  // 256
constexpr int BN = 256;
constexpr int BK = 32;      // K per pipeline stage (64-byte rows)
constexpr int STAGES = 4;   // LDS stage buffers; loads run 3 stages ahead
constexpr int NT = 512;     // 8 waves: 2 per SIMD
constexpr int SUPER = 8;  // m-tiles per supertile

constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 15) | (((n >> 4) & 3) << 14); }

__device__ __forceinline__ void dma16(const void* g, bf16* l) { __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0); }

// Compiler-level fence around the raw s_barrier (the barrier builtin itself
// does not order memory operations for the compiler).
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 4 direct loads (2 A, 2 B) per lane of one 32-wide K step into one stage
// buffer; load i of wave w fills the 16 rows (8i + w)*16 .. +16 (1 KB).
__device__ __forceinline__ void issue_stage(bf16* sa, bf16* sb, const bf16* abase, const uint32_t* aoff,
                                            const bf16* const* bbase, const uint32_t* boff, uint32_t k0, int wave) {
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16(abase + (aoff[i] + k0), sa + (8 * i + wave) * 512);
#pragma unroll
  for (int i = 0; i < 2; ++i) dma16(bbase[i] + (boff[i] + k0), sb + (8 * i + wave) * 512);
}

// LDS image of one stage: [row][4 chunks of 16 B], chunk c of row r at
// position c ^ ((r >> 2) & 3).  A half-wave reads 16 rows of one chunk; 64
// banks span four 64-byte rows, so the XOR spreads the 16 reads over all 16
// bank groups.
__device__ __forceinline__ int lds_pos(int r, int c) { return r * BK + ((c ^ ((r >> 2) & 3)) << 3); }

template <int NB>
__device__ __forceinline__ void load_frags(const bf16* sa, const bf16* sb, int ks, int wm, int wn, int lane,
                                           bf16x8* af, bf16x8* bfr) {
  const int c = ks * 2 + (lane >> 5);
#pragma unroll
  for (int ii = 0; ii < NB; ++ii) {
    const int rr = (wm + 2 * ii) * 32 + (lane & 31);
    af[ii] = *reinterpret_cast<const bf16x8*>(sa + lds_pos(rr, c));
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int rr = wn * 64 + jj * 32 + (lane & 31);
    bfr[jj] = *reinterpret_cast<const bf16x8*>(sb + lds_pos(rr, c));
  }
}

// MFMAs of one stage: 2 K sub-steps of 16, fragments double-buffered.
template <int NB>
__device__ __forceinline__ void compute_stage(f32x16 (&acc)[4][2], const bf16* sa, const bf16* sb, int wm, int wn,
                                              int lane) {
  bf16x8 af[2][NB], bfr[2][2];
  load_frags<NB>(sa, sb, 0, wm, wn, lane, af[0], bfr[0]);
  load_frags<NB>(sa, sb, 1, wm, wn, lane, af[1], bfr[1]);
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks)
#pragma unroll
    for (int ii = 0; ii < NB; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][ii], bfr[ks][jj], acc[ii][jj], 0, 0, 0);
}

// Four-stage direct-load pipeline over nk (a multiple of 4) K steps.  Per
// stage: wait for this wave's loads of the stage (two younger stages, 8
// loads, may stay in flight), one barrier (everyone's loads landed and
// everyone is done with the previous stage's buffer), refill that buffer
// three K steps ahead (the tail repeats the last K step; never read), MFMAs.
template <int NB>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[4][2], bf16* const* sA, bf16* const* sB, const bf16* abase,
                                         const uint32_t* aoff, const bf16* const* bbase, const uint32_t* boff,
                                         int nk, int wave, int wm, int wn, int lane) {
  const uint32_t klast = (uint32_t)(nk - 1) * BK;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) issue_stage(sA[st], sB[st], abase, aoff, bbase, boff, st * BK, wave);
  for (int kt = 0; kt < nk; kt += STAGES) {
#pragma unroll
    for (int st = 0; st < STAGES; ++st) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
      block_sync();
      const uint32_t kn = (uint32_t)(kt + st + STAGES - 1) * BK;
      const int nb = (st + STAGES - 1) % STAGES;
      issue_stage(sA[nb], sB[nb], abase, aoff, bbase, boff, kn < klast ? kn : klast, wave);
      compute_stage<NB>(acc, sA[st], sB[st], wm, wn, lane);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void gemm_big_kernel(FfnArgs f, int n_tiles_n, int list_begin_idx,
                                                         int list_end_idx) {
  __shared__ __attribute__((aligned(1024))) bf16 sA0[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA1[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA2[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sA3[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sB0[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sB1[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sB2[BN * BK];
  __shared__ __attribute__((aligned(1024))) bf16 sB3[BN * BK];
  bf16* const sA[STAGES] = {sA0, sA1, sA2, sA3};
  bf16* const sB[STAGES] = {sB0, sB1, sB2, sB3};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  const int mt_begin = list_begin_idx < 0 ? 0 : f.plan[list_begin_idx];
  const int mt_end = f.plan[list_end_idx];
  const int MT = mt_end - mt_begin;
  const int total = MT * n_tiles_n;
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  for (int it = 0;; ++it) {
    const int t = it * G + xcd * (G >> 3) + slot;
    if (t >= total) break;
    // supertile order: 8 m-tiles x all n-tiles, m fastest
    const int sbase = (t / (SUPER * n_tiles_n)) * SUPER;
    const int grp = MT - sbase < SUPER ? MT - sbase : SUPER;
    const int r = t - sbase * n_tiles_n;
    const int nt = r / grp;
    const int mt = mt_begin + sbase + r % grp;

    const int g = f.mt_group[mt];
    const int r0 = f.mt_row0[mt];
    const bool shared = g >= f.E;
    int base = 0, nrows;
    if (!shared) {
      base = f.offsets[g];
      nrows = f.offsets[g + 1] - base - r0;
    } else {
      nrows = f.T - r0;
    }
    nrows = nrows < BM ? nrows : BM;
    const int K = MODE == 1 ? f.H : (shared ? f.Is : f.I);
    const int Ncols = MODE == 1 ? (shared ? f.Is : f.I) : f.H;
    const int ncov = MODE == 1 ? BN / 2 : BN;
    if (nt * ncov >= Ncols) continue;

    // ---- sources of the 2 A and 2 B direct loads of each K step ----
    // load i of wave w fills LDS rows (8i + w)*16 .. +16 (1 KB); lane l ->
    // row +l/4, position l%4, so it fetches global chunk (l%4) ^ ((row>>2)&3)
    // = (l%4) ^ ((l>>4)&3).  Bases are wave-uniform (SGPRs); lanes carry
    // 32-bit element offsets.
    const int lrow = lane >> 2;
    const int gchunk = (lane & 3) ^ ((lane >> 4) & 3);
    const bf16* abase;
    if (MODE == 1) abase = reinterpret_cast<const bf16*>(f.x);
    else abase = shared ? reinterpret_cast<const bf16*>(f.h_sh) : reinterpret_cast<const bf16*>(f.h);
    uint32_t aoff[2], boff[2];
    const bf16* bbase[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int grp = 8 * i + wave;  // wave-uniform
      int rr = grp * 16 + lrow;
      rr = rr < nrows ? rr : nrows - 1;
      const int gr = base + r0 + rr;
      if (MODE == 1) {
        int tok = shared ? gr : f.sorted[gr] / f.k;
        tok = tok < f.T ? tok : f.T - 1;
        aoff[i] = (uint32_t)tok * (uint32_t)f.H + gchunk * 8;
      } else {
        aoff[i] = (uint32_t)gr * (uint32_t)K + gchunk * 8;
      }
      const int n = grp * 16 + lrow;  // B tile row
      int col;
      if (MODE == 1) {
        // tile rows: wave-column wc (64 rows) holds 32 gate rows then the 32
        // up rows of the same 32 hidden columns
        const bool up = ((grp * 16) & 63) >= 32;  // uniform per load
        col = nt * (BN / 2) + (n >> 6) * 32 + (n & 31);
        bbase[i] = shared ? reinterpret_cast<const bf16*>(up ? f.shu : f.shg)
                          : reinterpret_cast<const bf16*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg);
      } else {
        col = nt * BN + n;
        bbase[i] = shared ? reinterpret_cast<const bf16*>(f.shd) : reinterpret_cast<const bf16*>(f.wd) + (int64_t)g * f.sd;
      }
      col = col < Ncols ? col : Ncols - 1;
      boff[i] = (uint32_t)col * (uint32_t)K + gchunk * 8;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // M-blocks of 32 rows this wave computes (blocks wm, wm+2, ... below nrows)
    const int nblk_tile = (nrows + 31) / 32;
    const int nb = (nblk_tile - wm + 1) / 2;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // previous tile's stores settled before LDS reuse
    const int nk = K / BK;
    if (nb >= 4) mainloop<4>(acc, sA, sB, abase, aoff, bbase, boff, nk, wave, wm, wn, lane);
    else if (nb == 3) mainloop<3>(acc, sA, sB, abase, aoff, bbase, boff, nk, wave, wm, wn, lane);
    else if (nb == 2) mainloop<2>(acc, sA, sB, abase, aoff, bbase, boff, nk, wave, wm, wn, lane);
    else mainloop<1>(acc, sA, sB, abase, aoff, bbase, boff, nk, wave, wm, wn, lane);

    // ---- epilogue: C lane layout col = lane%32, row 8*(v/4) + 4*(lane/32) + v%4 ----
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int mb = wm + 2 * ii;
      if (mb * 32 >= nrows) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (rl >= nrows) continue;
        const int64_t gr = base + r0 + rl;
        if (MODE == 1) {
          const int col = nt * (BN / 2) + wn * 32 + (lane & 31);
          if (col < Ncols) {
            bf16* dst = shared ? reinterpret_cast<bf16*>(f.h_sh) + gr * f.Is : reinterpret_cast<bf16*>(f.h) + gr * f.I;
            dst[col] = f2bf(silu(acc[ii][0][v]) * acc[ii][1][v]);
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int col = nt * BN + wn * 64 + jj * 32 + (lane & 31);
            if (col < Ncols) {
              bf16* dst = shared ? reinterpret_cast<bf16*>(f.y_sh) : reinterpret_cast<bf16*>(f.y);
              dst[gr * f.H + col] = f2bf(acc[ii][jj][v]);
            }
          }
        }
      }
    }
  }
}

int big_grid() {
  static int g = 0;
  if (!g) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    g = (cus + 7) / 8 * 8;  // one workgroup per CU, a multiple of the 8 XCDs
  }
  return g;
}

}  // namespace

bool ffn_big_supported(const FfnArgs& a) {
  return !a.fp8 && a.H % (STAGES * BK) == 0 && a.I % (STAGES * BK) == 0 && (a.Is == 0 || a.Is % (STAGES * BK) == 0);
}

hipError_t launch_ffn_gemm_big(const FfnArgs& a, int phase, hipStream_t s) {
  const int wide = a.I > a.Is ? a.I : a.Is;
  const int ntn = phase == 1 ? (wide + BN / 2 - 1) / (BN / 2) : (a.H + BN - 1) / BN;
  if (phase == 1) gemm_big_kernel<1><<<big_grid(), NT, 0, s>>>(a, ntn, -1, 0);
  else gemm_big_kernel<2><<<big_grid(), NT, 0, s>>>(a, ntn, -1, 0);
  return hipGetLastError();
}

}  // namespace moe
