// Weight-streaming expert FFN for groups with few rows (decode, skew tails).
//
// When an expert holds only a handful of tokens the expert GEMMs of
// eq. expert(x) (Qwen3.8-Flash-Next study, MoE section) are bound by reading
// its weights once from HBM.  Here each wave owns one (16-row m-block,
// weight slab) item and streams the slab's weight rows straight from HBM into
// MFMA B fragments (v_mfma_f32_16x16x32_bf16: lane = weight row l%16, 8
// consecutive K values), with no LDS staging: every weight byte is used by
// exactly one wave.  The 16 activation rows (A fragments) come from L2.
// Loads for 8 K-steps are issued before their MFMAs so each lane keeps
// several 16-byte loads in flight.
//   gate/up item: 16 hidden columns (16 gate rows + 16 up rows), SiLU*mul in registers
//   down item   : 64 output columns (4 blocks of 16 W_down rows)
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int WAVES = 4;
constexpr int UNROLL = 8;
constexpr int KSTEP = 32;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int PHASE, bool FP8>
__global__ __launch_bounds__(WAVES * 64) void stream_kernel(FfnArgs f, int list_begin_idx, int list_end_idx) {
  constexpr int NB = PHASE == 1 ? 2 : 4;  // 16-column B blocks per item (gate+up, or 4 down blocks)
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int nw = gridDim.x * WAVES;
  const int sb_begin = list_begin_idx < 0 ? 0 : f.plan[list_begin_idx];
  const int sb_end = f.plan[list_end_idx];
  const int wide = PHASE == 1 ? (f.I > f.Is ? f.I : f.Is) : f.H;
  const int cols_per_item = PHASE == 1 ? 16 : 64;
  const int n_slabs = (wide + cols_per_item - 1) / cols_per_item;
  const int total = (sb_end - sb_begin) * n_slabs;
  const int m = lane & 15;       // A row / B column within a 16-block
  const int kq = (lane >> 4) * 8;  // K offset of this lane inside a 32-wide K step

  for (int item = gw; item < total; item += nw) {
    const int sb = sb_begin + item / n_slabs;
    const int slab = item % n_slabs;
    const int g = f.sb_group[sb];
    const int r0 = f.sb_row0[sb];
    const bool shared = g >= f.E;
    int base = 0, nrows;
    if (!shared) {
      base = f.offsets[g];
      nrows = f.offsets[g + 1] - base - r0;
    } else {
      nrows = f.T - r0;
    }
    nrows = nrows < 16 ? nrows : 16;
    const int K = PHASE == 1 ? f.H : (shared ? f.Is : f.I);
    const int Ncols = PHASE == 1 ? (shared ? f.Is : f.I) : f.H;
    const int c0 = slab * cols_per_item;
    if (c0 >= Ncols) continue;
    const bool fp8 = FP8 && !shared;

    // A row of this lane (zero when past the group's rows)
    const bf16* a_row = nullptr;
    if (m < nrows) {
      const int gr = base + r0 + m;
      if (PHASE == 1) {
        int tok = shared ? gr : f.sorted[gr] / f.k;
        tok = tok < f.T ? tok : f.T - 1;
        a_row = reinterpret_cast<const bf16*>(f.x) + (int64_t)tok * f.H;
      } else {
        a_row = shared ? reinterpret_cast<const bf16*>(f.h_sh) + (int64_t)gr * f.Is
                       : reinterpret_cast<const bf16*>(f.h) + (int64_t)gr * f.I;
      }
    }
    // B rows of this lane, one per 16-column block
    const void* b_row[NB];
    const float* s_row[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      int col = PHASE == 1 ? c0 + m : c0 + j * 16 + m;
      col = col < Ncols ? col : Ncols - 1;
      s_row[j] = nullptr;
      if (PHASE == 1) {
        const bool up = j == 1;
        if (shared) {
          b_row[j] = reinterpret_cast<const bf16*>(up ? f.shu : f.shg) + (int64_t)col * f.H;
        } else if (fp8) {
          b_row[j] = reinterpret_cast<const uint8_t*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg) +
                     (int64_t)col * f.H;
          const int kb = f.H / 128;
          s_row[j] = (up ? f.scu : f.scg) + (int64_t)g * (f.I / 128) * kb + (col / 128) * kb;
        } else {
          b_row[j] = reinterpret_cast<const bf16*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg) +
                     (int64_t)col * f.H;
        }
      } else {
        if (shared) {
          b_row[j] = reinterpret_cast<const bf16*>(f.shd) + (int64_t)col * f.Is;
        } else if (fp8) {
          b_row[j] = reinterpret_cast<const uint8_t*>(f.wd) + (int64_t)g * f.sd + (int64_t)col * f.I;
          const int kb = f.I / 128;
          s_row[j] = f.scd + (int64_t)g * (f.H / 128) * kb + (col / 128) * kb;
        } else {
          b_row[j] = reinterpret_cast<const bf16*>(f.wd) + (int64_t)g * f.sd + (int64_t)col * f.I;
        }
      }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = (K + KSTEP - 1) / KSTEP;
    for (int s0 = 0; s0 < nsteps; s0 += UNROLL) {
      u32x4 av[UNROLL];
      u32x4 bv[UNROLL][NB];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int kk = (s0 + u) * KSTEP + kq;
        const bool in = kk < K;
        av[u] = (in && a_row) ? ld16(a_row + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if (!in) {
            bv[u][j] = u32x4{0, 0, 0, 0};
          } else if (fp8) {
            const u32x2 c = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(b_row[j]) + kk);
            bv[u][j] = fp8x8_to_bf16x8(c, s_row[j][kk / 128]);
          } else {
            bv[u][j] = ld16(reinterpret_cast<const bf16*>(b_row[j]) + kk);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[u]), as_bf16x8(bv[u][j]), acc[j], 0, 0, 0);
    }

    // C fragment: lane holds column (lane & 15), rows 4*(lane>>4) + i.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (row >= nrows) continue;
      const int64_t gr = base + r0 + row;
      if (PHASE == 1) {
        const int col = c0 + m;
        if (col < Ncols) {
          bf16* dst = shared ? reinterpret_cast<bf16*>(f.h_sh) + gr * f.Is : reinterpret_cast<bf16*>(f.h) + gr * f.I;
          dst[col] = f2bf(silu(acc[0][i]) * acc[1][i]);
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

hipError_t launch_ffn_stream(const FfnArgs& a, int phase, hipStream_t s) {
  const int grid = stream_grid();
  const int blk = WAVES * 64;
  if (a.fp8) {
    if (phase == 1) stream_kernel<1, true><<<grid, blk, 0, s>>>(a, -1, 3);
    else stream_kernel<2, true><<<grid, blk, 0, s>>>(a, -1, 3);
    if (a.Is > 0) {
      if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, 3, 1);
      else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, 3, 1);
    }
  } else {
    if (phase == 1) stream_kernel<1, false><<<grid, blk, 0, s>>>(a, -1, 1);
    else stream_kernel<2, false><<<grid, blk, 0, s>>>(a, -1, 1);
  }
  return hipGetLastError();
}

}  // namespace moe
