// Weight-streaming work item of the streaming kernels: one wave contracts a
// group of at most 16 rows with one slab of an expert's weights, reading that
// slab from HBM exactly once (the expert GEMMs of eq. expert(x) in the
// Qwen3.8-Flash-Next study's MoE section are bound by that read when an
// expert holds few tokens).  Weights are loaded in long row runs into
// registers, re-laid into
// v_mfma_f32_16x16x32_bf16 fragments through a wave-private LDS stage (no
// barriers), and multiplied by the group's (at most 16) activation rows,
// which come from L2.  Each weight byte is read once, so the weight loads are
// non-temporal, which measured faster (16-token decode: gate/up 154 -> 142.5
// us, down 81 -> 73 us).  fp8 codes are decoded with their 128 x 128 block
// scale as fragments leave LDS.
//   gate/up item: 16 hidden columns (16 gate rows + 16 up rows), SiLU*mul in
//                 registers; SPLIT: 8 columns (8 gate + 8 up rows in one block)
//   down item   : 32 output columns (2 blocks of 16 W_down rows)
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace streamk {

constexpr int U = 4;  // K steps per batch
constexpr int KSTEP = 32;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

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
          wb[x][i] = ld16_nt(wrow0[half] + (live ? (uint32_t)(r * ldw + k) : 0u));
        } else {
          const int r = 2 * i + h < nvalid[j] ? 2 * i + h : nvalid[j] - 1;
          wb[x][j * 8 + i] = ld16_nt(wrow0[j] + (live ? (uint32_t)(r * ldw + k) : 0u));
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
// contiguous bytes.  Fragments are converted when read from LDS (8 codes to
// eight bf16, exactly), and each 128-wide K block's products are scaled by
// the rows' 128 x 128 block scale (s_row[j]: this lane's fragment row's scale
// row, indexed by k / 128) before they join the sums.
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
        wb[j * 4 + i] = ld16_nt(wrow0[j] + (uint32_t)(r * ldw + k));
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
  // A batch is two 128-wide K blocks.  The codes convert exactly to bf16
  // (every e4m3fn value is a bf16 value), the MFMAs of one K block add into
  // part[j], and part[j] times the block's scale goes into acc[j]: one
  // multiply-add per accumulator per K block instead of one multiply per
  // weight (the 16 rows of a block share one 128-row scale block).
  auto compute = [&](int x, int b) {
    const int n = lane & 15;
    const int hn = n & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 part[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = h * (NA / 2); s < (h + 1) * (NA / 2); ++s) {
        const int kk = kbeg + b * SB8 + s * KSTEP + kq;
        const u32x4 am = (a_row && kk < kend) ? av[x][s] : u32x4{0, 0, 0, 0};
        const int byte = s * KSTEP + kq;  // offset in the 256-byte row run
        const int cc = byte >> 4;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const u32x2 codes = *reinterpret_cast<const u32x2*>(lds + (j * 8 + (n >> 1)) * PAIR8 + hn * 256 +
                                                              ((cc ^ (hn << 3)) << 4) + (byte & 15));
          const u32x4 bv = fp8x8_to_bf16x8_exact(codes);
          part[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(am), as_bf16x8(bv), part[j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] += sc[x][j][h] * part[j];
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

// Bytes of wave-private LDS one item needs.
template <bool FP8, bool SPLIT>
constexpr int item_lds_bytes() {
  return (SPLIT ? 1 : 2) * 8 * (FP8 ? PAIR8 : PAIR);
}

// One item: slab `slab` of group g (routed expert g < E, or the shared
// expert g == E) for rows r0 .. r0+nrows-1 of the group (nrows <= 16), whose
// dispatched rows start at `base`.  The gathered token of each row: tok_row
// (the plan's list); else, when tok_mask is nonzero, the group's tokens as a
// bit mask (row m is the token of its m-th set bit: a batch of at most 32
// tokens whose dispatch is not in memory yet); else f.sorted.  lds: this
// wave's item_lds_bytes<FP8, SPLIT>() bytes.  Returns at once if the slab
// lies past the group's columns.
template <int PHASE, bool FP8, bool SPLIT>
__device__ __forceinline__ void stream_item(const FfnArgs& f, int g, int r0, int base, int nrows,
                                            const int32_t* tok_row, int slab, int lane, char* lds,
                                            uint32_t tok_mask = 0u) {
  static_assert(!SPLIT || (PHASE == 1 && !FP8), "split items are bf16 gate/up");
  constexpr int NB = SPLIT ? 1 : 2;
  const int cols_per_item = PHASE == 1 ? (SPLIT ? 8 : 16) : 32;
  const int m = lane & 15;  // A row / B column within a 16-block
  const bool shared = g >= f.E;
  const int K = PHASE == 1 ? f.H : (shared ? f.Is : f.I);
  const int Ncols = PHASE == 1 ? (shared ? f.Is : f.I) : f.H;
  const int c0 = slab * cols_per_item;
  if (c0 >= Ncols) return;

  // A row of this lane (zero when past the group's rows)
  const bf16* a_row = nullptr;
  if (m < nrows) {
    const int gr = base + r0 + m;
    if (PHASE == 1) {
      int tok;
      if (tok_row) {
        tok = tok_row[m];
      } else if (tok_mask) {
        uint32_t mm = tok_mask;
        for (int i = 0; i < m; ++i) mm &= mm - 1u;  // drop the m lowest set bits
        tok = __builtin_ctz(mm);
      } else {
        tok = g < f.E ? f.sorted[gr] / f.k : m;
      }
      tok = (unsigned)tok < (unsigned)f.T ? tok : f.T - 1;  // also clamps a negative index
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
    stream_dot_lds8<NB>(a_row, a_any, w0, nv, K, s_row, 0, K, lane, lds, acc);
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
    stream_dot_lds<NB, SPLIT, SPLIT ? 2 : 1>(a_row, a_any, w0, nv, K, 0, K, lane, lds, acc);
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

}  // namespace streamk
}  // namespace moe
