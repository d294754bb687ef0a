// Pipelined direct-load grouped expert GEMM for groups of hundreds of rows
// (MFMA-bound), gfx950: the gate/up and down contractions of eq. expert(x)
// in the Qwen3.8-Flash-Next study's MoE section (SwiGLU expert; "Per-expert
// FFN" in the pipeline figure), on v_mfma_f32_32x32x16_bf16.
//
// Tile 256 x 256, K step 32, 512 threads = 8 waves (two per SIMD, so one
// wave's MFMAs cover the other's LDS waits), each wave 128 x 64 (4 x 2 blocks
// of 32 x 32).  The kernel is a template over the tiling (tile size, wave
// grid, stages, workgroups per CU); a wave owns M-blocks {wm, wm + WM, ...}
// (interleaved, so a partial tile keeps every wave busy) and NJ consecutive
// N-blocks.  For gate/up the first half of a wave's N-blocks are gate rows
// and the second half the up rows of the same hidden columns, so SiLU(g) * u
// is formed in registers.
//
// Operands move HBM/L2 -> LDS with gfx950's direct loads (buffer_load ... lds
// through a buffer resource per operand, 16 bytes per lane, no VGPR staging)
// into statically separate stage buffers (A rows, then B rows), four stages,
// loads three K steps ahead and issued first in each step; waits are
// explicit s_waitcnt vmcnt + s_barrier.  The second K sub-step of a stage
// is carried (fp8: decoded first): its fragments are read during the first
// sub-step's MFMAs and its MFMAs run after the next barrier, while the next
// stage's first fragments are read, so no stage starts on an LDS wait.  A stage holds a 32-wide K slice,
// [row][4 chunks of 16 B], chunk c of row r at position c ^ ((r >> 2) & 3):
// a half-wave's 16-byte fragment reads cover 16 rows and 64 banks span four
// 64-byte rows, so the XOR spreads them over all banks.  (The template also
// takes a 64-wide K step: 8 chunks per 128-byte row, XOR (r >> 1) & 7.)  Each lane's direct
// load fetches the global chunk that belongs at its LDS position, so global
// reads stay whole 64-byte row segments.
//
// fp8 weights (e4m3 codes with 128 x 128 block scales): the B stage holds
// the codes, 32 bytes per row, laid out [16-byte chunk][row] within each
// 32-row block, so a fragment read (8 codes of one row) by 32 lanes touches
// 32 rows at a 16-byte stride.  The codes are decoded to bf16 with their
// block scale as fragments leave LDS; the tile's scales (one per 128-wide K
// block, for its gate and up row blocks or its two W_down row blocks) sit
// in a small LDS table.  With a 32-wide K step, stage step s uses K block s/4.
//
// Work: (group, 256-row m-tile) entries from the device plan; tiles are
// ordered in supertiles of a few m-tiles x all n-tiles and dealt to the
// persistent grid so that consecutive tiles land on one XCD (workgroup i runs
// on XCD i mod 8), sharing A slices and weight slices in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {


template <int BM_, int BN_, int WM_, int WN_, int S_, int WG_PER_CU_, int BK_ = 32, bool F8_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_, BK = BK_;
  static constexpr bool F8 = F8_;       // B holds fp8 codes (1 byte per element)
  static constexpr int RPL = 512 / BK;  // rows one 1 KB direct load fills
  static constexpr int RPL8 = 1024 / BK;  // fp8 B rows one 1 KB direct load fills
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WAVES_PER_EU = NW * WG_PER_CU_ / 4;
  static constexpr int WG_PER_CU = WG_PER_CU_;
  static constexpr int MI = BM / (32 * WM);  // M-blocks per wave
  static constexpr int NJ = BN / (32 * WN);  // N-blocks per wave
  static constexpr int CW = NJ * 32;         // B tile rows per wave column
  static constexpr int LA = BM / (RPL * NW);  // A direct loads per lane per stage
  static constexpr int LB = F8 ? BN / (RPL8 * NW) : BN / (RPL * NW);  // B direct loads per lane per stage
  static constexpr int L = LA + LB;
  static constexpr int STAGE = (BM + BN) * BK;  // elements per stage buffer
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(MI >= 1 && NJ >= 2 && NJ % 2 == 0 && LA >= 1 && LB >= 1, "tiling");
  static_assert(S >= 2 && S <= 6 && L * (S - 2) < 64, "pipeline depth");
  static_assert(S * STAGE * 2 * WG_PER_CU_ <= 160 * 1024, "LDS");
  static_assert(!F8 || (BK == 32 && S == 4 && MI * NJ <= 8 && NJ == 2 && CW == 64), "fp8 B tiling");
};
using BigCfg = Cfg<256, 256, 2, 4, 4, 1>;
using BigCfg8 = Cfg<256, 256, 2, 4, 4, 1, 32, true>;

constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 15) | (((n >> 4) & 3) << 14); }
// the same wait, and for every LDS operation of this wave
constexpr int vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~0xF00; }

// A 16-byte direct load (global memory to LDS, no registers) through a
// buffer resource over base, at byte offset voff + soff < 2^32 (the layer
// checks keep every element offset below 2^31); soff is wave-uniform (the K
// step), voff the lane's row and chunk.  The compiler counts buffer loads to LDS
// apart from LDS reads, so fragment reads keep partial LDS waits; with the
// global_load_lds form in flight it waits for every outstanding LDS operation
// before each MFMA that consumes a fragment.
constexpr int kBufferFlags = 0x00020000;  // raw (untyped) 32-bit buffer access
__device__ __forceinline__ void dma16b(const void* base, uint32_t voff, uint32_t soff, bf16* l) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xFFFFFFFF,
                                                                      kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, voff, soff, 0, 0);
}

// Compiler-level fence around the raw s_barrier (the barrier builtin itself
// does not order memory operations for the compiler).
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk c of row r: 4 chunks per 64-byte row XOR (r >> 2) & 3, or 8 per
// 128-byte row XOR (r >> 1) & 7 (16 rows of one chunk hit 16 bank groups).
template <int BK>
__device__ __forceinline__ int swz(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
template <int BK>
__device__ __forceinline__ int lds_pos(int r, int c) { return r * BK + ((c ^ swz<BK>(r)) << 3); }

// The direct loads of one K step into one stage buffer: load i of wave w
// fills 16 rows (NW*i + w)*16 .. +16 (1 KB) of the A part, then of the B part.
template <class C>
__device__ __forceinline__ void issue_stage(bf16* st, const bf16* abase, const uint32_t* aoff,
                                            const bf16* const* bbase, const uint32_t* boff, uint32_t k0, int wave) {
#pragma unroll
  for (int i = 0; i < C::LA; ++i) dma16b(abase, aoff[i] * 2u, k0 * 2u, st + (C::NW * i + wave) * 512);
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    // fp8: bbase holds byte pointers, boff byte offsets (k0 counts codes)
    if constexpr (C::F8)
      dma16b(bbase[i], boff[i], k0, st + C::BM * C::BK + (C::NW * i + wave) * 512);
    else
      dma16b(bbase[i], boff[i] * 2u, k0 * 2u, st + C::BM * C::BK + (C::NW * i + wave) * 512);
  }
}

// Element offsets of this lane's fragment reads inside a stage for K sub-step
// ks: row (lane % 32) of the wave's first A / B block, chunk 2*ks + lane/32,
// swizzled.  Block ii / jj adds a whole number of 32-row blocks, so every
// fragment read is one of these plus a compile-time offset.
struct FragOff {
  int a[4], b[4];  // per 16-wide K sub-step of a stage
  int b8;          // fp8 B: byte offset of this lane's first code (block 0, chunk 0)
};

template <class C>
__device__ __forceinline__ FragOff frag_offsets(int wm, int wn, int lane) {
  FragOff o;
#pragma unroll
  for (int ks = 0; ks < C::BK / 16; ++ks) {
    const int c = ks * 2 + (lane >> 5);
    o.a[ks] = lds_pos<C::BK>(wm * 32 + (lane & 31), c);
    o.b[ks] = lds_pos<C::BK>(C::BM + wn * C::CW + (lane & 31), c);
  }
  o.b8 = C::BM * C::BK * 2 + wn * (C::CW / 32) * 1024 + (lane & 31) * 16 + 8 * (lane >> 5);
  return o;
}

template <class C, int NB>
__device__ __forceinline__ void load_frags(const bf16* st, int ks, const FragOff& o, bf16x8* af, bf16x8* bfr) {
#pragma unroll
  for (int ii = 0; ii < NB; ++ii)
    af[ii] = *reinterpret_cast<const bf16x8*>(st + o.a[ks] + ii * C::WM * 32 * C::BK);
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj)
    bfr[jj] = *reinterpret_cast<const bf16x8*>(st + o.b[ks] + jj * 32 * C::BK);
}

// bf16 fragments of one K sub-step held across a barrier: the stage's second
// sub-step, whose MFMAs run at the start of the next stage (zero at a tile's
// first stage, so there they add nothing).
template <class C>
constexpr bool kCarry = C::BK == 32 && C::MI * C::NJ <= 8;

template <class C, int NB>
struct Carry {
  bf16x8 a[NB], b[C::NJ];
};

template <class C, int NB>
__device__ __forceinline__ void mfma_sub(f32x16 (&acc)[C::MI][C::NJ], const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
  for (int ii = 0; ii < NB; ++ii)
#pragma unroll
    for (int jj = 0; jj < C::NJ; ++jj)
      acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ii], bfr[jj], acc[ii][jj], 0, 0, 0);
}

// bf16 stage with the second sub-step carried: the first sub-step's fragment
// reads run under the previous stage's carried MFMAs, the second sub-step's
// reads under the first sub-step's MFMAs, so no stage starts on an LDS wait.
template <class C, int NB>
__device__ __forceinline__ void compute_stage_carry(f32x16 (&acc)[C::MI][C::NJ], const bf16* st, const FragOff& o,
                                                    Carry<C, NB>& cy) {
  static_assert(C::BK == 32 && !C::F8, "two bf16 K sub-steps per stage");
  bf16x8 af[NB], bfr[C::NJ];
  load_frags<C, NB>(st, 0, o, af, bfr);
  mfma_sub<C, NB>(acc, cy.a, cy.b);
  mfma_sub<C, NB>(acc, af, bfr);
  load_frags<C, NB>(st, 1, o, cy.a, cy.b);
  constexpr int NR = NB + C::NJ;  // fragment reads per sub-step
  constexpr int NM = NB * C::NJ;  // MFMAs per sub-step
  constexpr int NP = NR < NM ? NR : NM;
  // the stage's direct loads (issued just before) go out first, for the
  // longest lead
  __builtin_amdgcn_sched_group_barrier(0x010, C::L, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
    if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
  }
}

// fp8 stage with the second sub-step carried, as above: the carried
// fragments are decoded (with this stage's block scales) before they are
// carried.  B block jj: 8 codes of row (lane % 32) at K 16*ks + 8*(lane/32),
// in chunk ks of its 32-row block; block 0 takes scale sc0, block 1 sc1.
template <class C, int NB>
__device__ __forceinline__ void compute_stage_carry8(f32x16 (&acc)[C::MI][C::NJ], const bf16* st, const FragOff& o,
                                                     float sc0, float sc1, Carry<C, NB>& cy) {
  static_assert(C::BK == 32 && C::F8, "two fp8 K sub-steps per stage");
  const char* sb = reinterpret_cast<const char*>(st) + o.b8;
  bf16x8 af[NB], bfr[C::NJ];
  u32x2 c0[C::NJ], c1[C::NJ];
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) c0[jj] = *reinterpret_cast<const u32x2*>(sb + jj * 1024);
#pragma unroll
  for (int ii = 0; ii < NB; ++ii) af[ii] = *reinterpret_cast<const bf16x8*>(st + o.a[0] + ii * C::WM * 32 * C::BK);
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj)
    bfr[jj] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(c0[jj], jj == 0 ? sc0 : sc1));
  mfma_sub<C, NB>(acc, cy.a, cy.b);
  mfma_sub<C, NB>(acc, af, bfr);
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj) c1[jj] = *reinterpret_cast<const u32x2*>(sb + jj * 1024 + 512);
#pragma unroll
  for (int ii = 0; ii < NB; ++ii) cy.a[ii] = *reinterpret_cast<const bf16x8*>(st + o.a[1] + ii * C::WM * 32 * C::BK);
#pragma unroll
  for (int jj = 0; jj < C::NJ; ++jj)
    cy.b[jj] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(c1[jj], jj == 0 ? sc0 : sc1));
  // Schedule: direct loads first; the carried MFMAs with the first
  // sub-step's reads, then its decode over their second half; the first
  // sub-step's MFMAs with the second sub-step's reads and decode likewise.
  constexpr int NR = NB + C::NJ;  // fragment reads per sub-step
  constexpr int NM = NB * C::NJ;  // MFMAs per sub-step
  constexpr int NV = 16 * C::NJ;  // decode instructions per sub-step
  constexpr int NH = NM - NM / 2; // MFMAs that the decode spreads over
  __builtin_amdgcn_sched_group_barrier(0x010, C::L, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i >= NM / 2) __builtin_amdgcn_sched_group_barrier(0x002, NV / NH, 0);
    }
    if constexpr (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
  }
}

// MFMAs of one stage: 2 K sub-steps of 16, fragments of both loaded first.
template <class C, int NB>
__device__ __forceinline__ void compute_stage(f32x16 (&acc)[C::MI][C::NJ], const bf16* st, const FragOff& o,
                                              float sc0, float sc1) {
  if constexpr (C::F8) {
    // B block jj: 8 codes of row (lane % 32) at K 16*ks + 8*(lane/32), in
    // chunk ks of its 32-row block; block 0 takes scale sc0, block 1 sc1
    // (one K sub-step at a time: the decode's temporaries leave no room for
    // both sub-steps' fragments next to the 128 accumulators)
    const char* sb = reinterpret_cast<const char*>(st) + o.b8;
    constexpr int KS = C::BK / 16;
    bf16x8 af[KS][NB], bfr[KS][C::NJ];
    u32x2 codes[KS][C::NJ];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj) codes[ks][jj] = *reinterpret_cast<const u32x2*>(sb + jj * 1024 + ks * 512);
#pragma unroll
      for (int ii = 0; ii < NB; ++ii)
        af[ks][ii] = *reinterpret_cast<const bf16x8*>(st + o.a[ks] + ii * C::WM * 32 * C::BK);
#pragma unroll
      for (int jj = 0; jj < C::NJ; ++jj)
        bfr[ks][jj] = __builtin_bit_cast(bf16x8, fp8x8_to_bf16x8(codes[ks][jj], jj == 0 ? sc0 : sc1));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int ii = 0; ii < NB; ++ii)
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][ii], bfr[ks][jj], acc[ii][jj], 0, 0, 0);
    // Schedule as in the bf16 path, with each sub-step's decode (VALU) placed
    // among the previous sub-step's MFMAs.
    constexpr int NR = NB + C::NJ;  // fragment reads per sub-step
    constexpr int NM = NB * C::NJ;  // MFMAs per sub-step
    constexpr int NV = 16 * C::NJ;  // decode instructions per sub-step
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV / NM, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  } else if constexpr (C::MI * C::NJ > 8) {
    // 128 x 128 wave tiles: one K sub-step of fragments at a time
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) {
      bf16x8 af[NB], bfr[C::NJ];
      load_frags<C, NB>(st, ks, o, af, bfr);
#pragma unroll
      for (int ii = 0; ii < NB; ++ii)
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ii], bfr[jj], acc[ii][jj], 0, 0, 0);
    }
  } else {
    bf16x8 af[C::BK / 16][NB], bfr[C::BK / 16][C::NJ];
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks) load_frags<C, NB>(st, ks, o, af[ks], bfr[ks]);
#pragma unroll
    for (int ks = 0; ks < C::BK / 16; ++ks)
#pragma unroll
      for (int ii = 0; ii < NB; ++ii)
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][ii], bfr[ks][jj], acc[ii][jj], 0, 0, 0);
    // Schedule: sub-step 0's fragment reads, then each sub-step's MFMAs
    // alternating with the next sub-step's reads, so LDS latency hides under
    // MFMAs (left alone, the compiler reuses one set of fragment registers
    // and waits on LDS before every few MFMAs).
    constexpr int NR = NB + C::NJ;  // fragment reads per sub-step
    constexpr int NM = NB * C::NJ;  // MFMAs per sub-step
    constexpr int NP = NR < NM ? NR : NM;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ks = 0; ks + 1 < C::BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
      if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

// One K step s held in buffer b: wait until this wave's loads of step s have
// landed (the S-2 younger stages may stay in flight), one barrier (every
// wave's loads landed, every wave done with buffer b-1), refill buffer b-1
// with step s+S-1 (past the end: the last step again, never read), MFMAs.
// fp8: sc0 / sc1 are this wave's two LDS scale rows (indexed by K block);
// with four stages of 32-wide K steps, stage 0 starts each 128-wide K block,
// where the block's two scales are read into scl0 / scl1.
template <class C, int NB, int B>
__device__ __forceinline__ void step(f32x16 (&acc)[C::MI][C::NJ], bf16* const* stg, const bf16* abase,
                                     const uint32_t* aoff, const bf16* const* bbase, const uint32_t* boff, int s,
                                     uint32_t klast, int wave, const FragOff& o, const float* sc0,
                                     const float* sc1, float& scl0, float& scl1, Carry<C, NB>& cy) {
  if constexpr (C::F8 && B == 0) {
    scl0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc0[s >> 2])));
    scl1 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc1[s >> 2])));
  }
  // carried reads of buffer b-1 must be done before any wave refills it
  if constexpr (kCarry<C>) {
    // nothing of the previous stage (its last MFMAs cover its last reads)
    // moves past the wait and barrier
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((C::S - 2) * C::L));
    block_sync();
    __builtin_amdgcn_sched_barrier(0);
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((C::S - 2) * C::L));
    block_sync();
  }
  const uint32_t kn = (uint32_t)(s + C::S - 1) * C::BK;
  issue_stage<C>(stg[(B + C::S - 1) % C::S], abase, aoff, bbase, boff, kn < klast ? kn : klast, wave);
  if constexpr (kCarry<C> && C::F8) compute_stage_carry8<C, NB>(acc, stg[B], o, scl0, scl1, cy);
  else if constexpr (kCarry<C>) compute_stage_carry<C, NB>(acc, stg[B], o, cy);
  else compute_stage<C, NB>(acc, stg[B], o, scl0, scl1);
}

// The K loop of one tile over nk steps, nk % S == R: step s uses buffer s % S.
template <class C, int NB, int R>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[C::MI][C::NJ], bf16* const* stg, const bf16* abase,
                                         const uint32_t* aoff, const bf16* const* bbase, const uint32_t* boff,
                                         int nk, int wave, const FragOff& o, const float* sc0, const float* sc1) {
  const uint32_t klast = (uint32_t)(nk - 1) * C::BK;
  float scl0 = 0.f, scl1 = 0.f;  // fp8: the current K block's scales
  Carry<C, NB> cy;
#pragma unroll
  for (int i = 0; i < NB; ++i) cy.a[i] = bf16x8{};
#pragma unroll
  for (int j = 0; j < C::NJ; ++j) cy.b[j] = bf16x8{};
  // every wave's loads (vmcnt(0) before the call) and LDS reads of the
  // previous tile are finished before its buffers are refilled
  block_sync();
#pragma unroll
  for (int st = 0; st < C::S - 1; ++st) {
    const uint32_t k0 = (uint32_t)st * C::BK;
    issue_stage<C>(stg[st], abase, aoff, bbase, boff, k0 < klast ? k0 : klast, wave);
  }
  const int nfull = nk - R;
  for (int kt = 0; kt < nfull; kt += C::S) {
    step<C, NB, 0>(acc, stg, abase, aoff, bbase, boff, kt + 0, klast, wave, o, sc0, sc1, scl0, scl1, cy);
    step<C, NB, 1>(acc, stg, abase, aoff, bbase, boff, kt + 1, klast, wave, o, sc0, sc1, scl0, scl1, cy);
    if constexpr (C::S > 2) step<C, NB, 2>(acc, stg, abase, aoff, bbase, boff, kt + 2, klast, wave, o, sc0, sc1, scl0, scl1, cy);
    if constexpr (C::S > 3) step<C, NB, 3>(acc, stg, abase, aoff, bbase, boff, kt + 3, klast, wave, o, sc0, sc1, scl0, scl1, cy);
    if constexpr (C::S > 4) step<C, NB, 4>(acc, stg, abase, aoff, bbase, boff, kt + 4, klast, wave, o, sc0, sc1, scl0, scl1, cy);
    if constexpr (C::S > 5) step<C, NB, 5>(acc, stg, abase, aoff, bbase, boff, kt + 5, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  }
  if constexpr (R > 0) step<C, NB, 0>(acc, stg, abase, aoff, bbase, boff, nfull + 0, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  if constexpr (R > 1) step<C, NB, 1>(acc, stg, abase, aoff, bbase, boff, nfull + 1, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  if constexpr (R > 2) step<C, NB, 2>(acc, stg, abase, aoff, bbase, boff, nfull + 2, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  if constexpr (R > 3) step<C, NB, 3>(acc, stg, abase, aoff, bbase, boff, nfull + 3, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  if constexpr (R > 4) step<C, NB, 4>(acc, stg, abase, aoff, bbase, boff, nfull + 4, klast, wave, o, sc0, sc1, scl0, scl1, cy);
  if constexpr (kCarry<C>) mfma_sub<C, NB>(acc, cy.a, cy.b);
}

template <class C, int NB>
__device__ __forceinline__ void mainloop_r(f32x16 (&acc)[C::MI][C::NJ], bf16* const* stg, const bf16* abase,
                                           const uint32_t* aoff, const bf16* const* bbase, const uint32_t* boff,
                                           int nk, int wave, const FragOff& o, const float* sc0, const float* sc1) {
  const int r = nk % C::S;
  if (r == 0) mainloop<C, NB, 0>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
  else if (C::S > 1 && r == 1) mainloop<C, NB, 1 % C::S>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
  else if (C::S > 2 && r == 2) mainloop<C, NB, 2 % C::S>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
  else if (C::S > 3 && r == 3) mainloop<C, NB, 3 % C::S>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
  else if (C::S > 4 && r == 4) mainloop<C, NB, 4 % C::S>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
  else mainloop<C, NB, 5 % C::S>(acc, stg, abase, aoff, bbase, boff, nk, wave, o, sc0, sc1);
}

// One 256 x 256 output tile: m-tile mt (a list entry of the plan: group and
// first row) x n-tile nt.  stg: the S stage buffers; ssc: fp8 scale table.
// A tile with fewer rows than BM computes only its M-blocks (a wave with none
// computes block wm on rows it never stores), and its A loads of 16-row
// groups past the last row read one 16-byte chunk for all lanes (those LDS
// rows are never stored).
template <class C, int MODE>
__device__ __forceinline__ void run_tile(const FfnArgs& f, int mt, int nt, bf16* const* stg, float* ssc, int tid,
                                         int lane, int wave, const FragOff& fo) {
  const int wm = wave / C::WN, wn = wave % C::WN;
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
  nrows = nrows < C::BM ? nrows : C::BM;
  const int K = MODE == 1 ? f.H : (shared ? f.Is : f.I);
  const int Ncols = MODE == 1 ? (shared ? f.Is : f.I) : f.H;
  const int ncov = MODE == 1 ? C::BN / 2 : C::BN;
  if (nt * ncov >= Ncols) return;

  // ---- sources of the direct loads of each K step ----
  // load i of wave w fills rows (NW*i + w)*RPL .. +RPL of its part; lane l
  // lands at row +l/(BK/8), position l%(BK/8), so it fetches the global
  // chunk that belongs there: position ^ swz(row).  Bases are wave-uniform
  // (SGPRs); lanes carry 32-bit element offsets.
  constexpr int LPR = C::BK / 8;  // lanes per row
  const int lrow = lane / LPR;
  const int lpos = lane % LPR;
  const bf16* abase;
  if (MODE == 1) abase = reinterpret_cast<const bf16*>(f.x);
  else abase = shared ? reinterpret_cast<const bf16*>(f.h_sh) : reinterpret_cast<const bf16*>(f.h);
  uint32_t aoff[C::LA], boff[C::LB];
  const bf16* bbase[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int row = (C::NW * i + wave) * C::RPL + lrow;
    // a load whose rows all lie past the tile's: every lane reads the same
    // 16 bytes (one cache line request instead of sixteen; the loads stay
    // unconditional, so the compiler's wait counts stay exact)
    const bool dead = (C::NW * i + wave) * C::RPL >= nrows;
    const int gchunk = dead ? 0 : lpos ^ swz<C::BK>(row);
    const int rr = dead ? nrows - 1 : (row < nrows ? row : nrows - 1);
    const int gr = base + r0 + rr;
    if (MODE == 1) {
      int tok = shared ? gr : f.sorted[gr] / f.k;
      tok = (unsigned)tok < (unsigned)f.T ? tok : f.T - 1;  // also clamps a negative index
      aoff[i] = (uint32_t)tok * (uint32_t)f.H + gchunk * 8;
    } else {
      aoff[i] = (uint32_t)gr * (uint32_t)K + gchunk * 8;
    }
  }
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    if constexpr (C::F8) {
      // load i of wave w fills B rows (NW*i + w)*32 .. +32 as [chunk][row]:
      // lane l takes row +l%32, 16-byte chunk l/32 of the 32-code K slice
      const int grow0 = (C::NW * i + wave) * C::RPL8;
      const int n = grow0 + (lane & 31);
      const int ch = lane >> 5;
      int col;
      const uint8_t* mat;
      if (MODE == 1) {
        const bool up = (grow0 % C::CW) >= C::CW / 2;
        col = nt * (C::BN / 2) + (n / C::CW) * (C::CW / 2) + (n % (C::CW / 2));
        mat = reinterpret_cast<const uint8_t*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg);
      } else {
        col = nt * C::BN + n;
        mat = reinterpret_cast<const uint8_t*>(f.wd) + (int64_t)g * f.sd;
      }
      col = col < Ncols ? col : Ncols - 1;
      bbase[i] = reinterpret_cast<const bf16*>(mat);
      boff[i] = (uint32_t)col * (uint32_t)K + ch * 16;
    } else {
      const int grow0 = (C::NW * i + wave) * C::RPL;  // wave-uniform first row of the load
      const int n = grow0 + lrow;                       // B tile row
      const int gchunk = lpos ^ swz<C::BK>(n);
      int col;
      if (MODE == 1) {
        // wave column wc (CW rows) holds CW/2 gate rows, then the up rows of
        // the same CW/2 hidden columns
        const bool up = (grow0 % C::CW) >= C::CW / 2;
        col = nt * (C::BN / 2) + (n / C::CW) * (C::CW / 2) + (n % (C::CW / 2));
        bbase[i] = shared ? reinterpret_cast<const bf16*>(up ? f.shu : f.shg)
                          : reinterpret_cast<const bf16*>(up ? f.wu : f.wg) + (int64_t)g * (up ? f.su : f.sg);
      } else {
        col = nt * C::BN + n;
        bbase[i] = shared ? reinterpret_cast<const bf16*>(f.shd) : reinterpret_cast<const bf16*>(f.wd) + (int64_t)g * f.sd;
      }
      col = col < Ncols ? col : Ncols - 1;
      boff[i] = (uint32_t)col * (uint32_t)K + gchunk * 8;
    }
  }

  // fp8: the tile's block scales, K block kb of row sel at ssc[sel*nkb + kb]
  // (gate/up: sel 0 gate, 1 up, of hidden block nt; down: W_down row
  // blocks 2nt and 2nt+1, the second clamped at the last)
  const float* sc0 = nullptr;
  const float* sc1 = nullptr;
  if constexpr (C::F8) {
    const int nkb = K / 128;
    for (int t = tid; t < 2 * nkb; t += C::NT) {
      const int sel = t / nkb, kb = t - sel * nkb;
      float v;
      if (MODE == 1) {
        v = (sel ? f.scu : f.scg)[((int64_t)g * (f.I / 128) + nt) * nkb + kb];
      } else {
        int rb = 2 * nt + sel;
        rb = rb < f.H / 128 ? rb : f.H / 128 - 1;
        v = f.scd[((int64_t)g * (f.H / 128) + rb) * nkb + kb];
      }
      ssc[t] = v;
    }
    if (MODE == 1) {
      sc0 = ssc;
      sc1 = ssc + nkb;
    } else {
      sc0 = sc1 = ssc + (wn * C::CW / 128) * nkb;
    }
  }

  f32x16 acc[C::MI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::MI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // M-blocks of 32 rows this wave computes (blocks wm, wm+WM, ... below nrows)
  const int nblk_tile = (nrows + 31) / 32;
  const int nb = (nblk_tile - wm + C::WM - 1) / C::WM;
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // previous tile's loads and stores settled
  const int nk = K / C::BK;
  if constexpr (C::MI >= 4) {
    if (nb >= 4) mainloop_r<C, 4>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
    else if (nb == 3) mainloop_r<C, 3>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
    else if (nb == 2) mainloop_r<C, 2>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
    else mainloop_r<C, 1>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
  } else {
    if (nb >= 2) mainloop_r<C, 2>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
    else mainloop_r<C, 1>(acc, stg, abase, aoff, bbase, boff, nk, wave, fo, sc0, sc1);
  }

  // ---- epilogue through LDS ----
  // The tile leaves in M bands of WM*32 rows: band ii (M-blocks WM*ii ..
  // WM*ii + WM-1) goes, as bf16 (gate/up: SiLU(g)*u), into the stage
  // buffers (BPS bands each), then every thread stores whole 16-byte row
  // chunks.  C lane layout of a
  // 32x32 block: col = lane%32, row 8*(v/4) + 4*(lane/32) + v%4.  Chunk c of
  // band row r sits at c ^ (4 * ((r >> 2) & 1)), so the two half-waves'
  // rows (4 apart) write different banks.
  constexpr int CCOLS = MODE == 1 ? C::BN / 2 : C::BN;  // output columns of the tile
  constexpr int CPR = CCOLS / 8;                        // 16-byte chunks per row
  constexpr int BAND = C::WM * 32;
  constexpr int BPS = C::STAGE / (BAND * CCOLS);        // bands per stage buffer
  static_assert(BPS >= 1 && C::MI <= C::S * BPS && CPR >= 8, "epilogue staging");
  auto cpos = [&](int r, int col) { return r * CCOLS + ((((col >> 3) ^ (((r >> 2) & 1) << 2))) << 3) + (col & 7); };
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // trailing (redundant) direct loads have landed
  block_sync();                              // every wave is done reading the stage buffers
#pragma unroll
  for (int ii = 0; ii < C::MI; ++ii) {
    bf16* ct = stg[ii / BPS] + (ii % BPS) * BAND * CCOLS;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if constexpr (MODE == 1) {
#pragma unroll
        for (int jj = 0; jj < C::NJ / 2; ++jj)
          ct[cpos(r, wn * (C::CW / 2) + jj * 32 + (lane & 31))] =
              f2bf(silu(acc[ii][jj][v]) * acc[ii][jj + C::NJ / 2][v]);
      } else {
#pragma unroll
        for (int jj = 0; jj < C::NJ; ++jj) ct[cpos(r, wn * C::CW + jj * 32 + (lane & 31))] = f2bf(acc[ii][jj][v]);
      }
    }
  }
  block_sync();
  bf16* obase;
  int ld;
  if (MODE == 1) {
    obase = shared ? reinterpret_cast<bf16*>(f.h_sh) : reinterpret_cast<bf16*>(f.h);
    ld = shared ? f.Is : f.I;
  } else {
    obase = shared ? reinterpret_cast<bf16*>(f.y_sh) : reinterpret_cast<bf16*>(f.y);
    ld = f.H;
  }
#pragma unroll
  for (int ii = 0; ii < C::MI; ++ii) {
    const bf16* ct = stg[ii / BPS] + (ii % BPS) * BAND * CCOLS;
    for (int q = tid; q < BAND * CPR; q += C::NT) {
      const int r = q / CPR, c = q % CPR;
      const int trow = ii * BAND + r;  // band ii holds tile rows ii*BAND ..
      const int col = nt * CCOLS + c * 8;
      if (trow < nrows && col < Ncols)
        st16(obase + (int64_t)(base + r0 + trow) * ld + col, ld16(ct + cpos(r, c * 8)));
    }
  }
}

// The persistent phase kernel: the phase's GEMM tiles (m-tiles
// [plan[tb], plan[te]) x n-tiles, ragged last m-tiles included), dealt to
// XCDs in the static order of supertiles of `super` m-tiles x all n-tiles:
// workgroup i runs on XCD i % 8, and XCD x takes tiles [x * chunk, (x+1) *
// chunk) of every round of G tiles (chunk = G / 8), so the tiles it runs at
// the same time share A and weight slices in its L2.  Its workgroups claim
// those tiles in order through the XCD's counter, so a workgroup that drew a
// ragged (cheaper) tile takes the next one sooner; a workgroup whose XCD has
// run out moves on to the next XCD's counter.  counters: 8 ints, zero at
// launch.
template <class C, int MODE>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void ffn_tiles_kernel(FfnArgs f, int n_tiles_n, int super,
                                                                           int tb, int te, int32_t* counters,
                                                                           int reserve) {
  __shared__ __attribute__((aligned(1024))) bf16 s0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 s1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) bf16 s2[C::S > 2 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16 s3[C::S > 3 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16 s4[C::S > 4 ? C::STAGE : 8];
  __shared__ __attribute__((aligned(1024))) bf16 s5[C::S > 5 ? C::STAGE : 8];
  __shared__ float ssc[C::F8 ? 256 : 1];  // fp8: two rows of K-block scales
  __shared__ int claim[2];
  // separate arrays: the compiler then knows that a fragment read from one
  // buffer does not wait on the direct loads in flight into the others
  bf16* const stg[6] = {s0, s1, s2, s3, s4, s5};
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const FragOff fo = frag_offsets<C>(wave / C::WN, wave % C::WN, lane);

  const int mt_first = tb == kPlanStart ? 0 : f.plan[tb];
  const int MT = f.plan[te] - mt_first;
  const int total = MT * n_tiles_n;
  // With streaming work in the plan and a streaming launch running beside
  // this one, the last `reserve` workgroups (a multiple of 8, so every XCD
  // gives up the same number) leave at once and free their CUs for it.
  const int G = reserve > 0 && f.plan[kPlanBlocks] > 0 ? (int)gridDim.x - reserve : (int)gridDim.x;
  if ((int)blockIdx.x >= G) return;
  const int chunk = G >> 3;
  auto xcd_tiles = [&](int x) {
    return (total / G) * chunk + min(max(total % G - x * chunk, 0), chunk);
  };

  int victim = blockIdx.x & 7;  // the XCD whose counter this workgroup claims from
  int tried = 0;
  for (;;) {
    if (tid == 0) {
      int xv = -1, c = 0;
      while (tried < 8) {
        const int tx = xcd_tiles(victim);
        if (tx > 0) {
          c = atomicAdd(&counters[victim], 1);
          if (c < tx) {
            xv = victim;
            break;
          }
        }
        victim = (victim + 1) & 7;
        ++tried;
      }
      claim[0] = xv;
      claim[1] = c;
    }
    __syncthreads();
    const int xv = claim[0], c = claim[1];
    __syncthreads();  // claim[] may be rewritten for the next tile
    if (xv < 0) break;
    const int t = (c / chunk) * G + xv * chunk + c % chunk;
    // supertile order: `super` m-tiles x all n-tiles, m fastest
    const int sbase = (t / (super * n_tiles_n)) * super;
    const int grp = MT - sbase < super ? MT - sbase : super;
    const int r = t - sbase * n_tiles_n;
    run_tile<C, MODE>(f, mt_first + sbase + r % grp, r / grp, stg, ssc, tid, lane, wave, fo);
  }
}

int cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return cus;
}

// One launch of a phase over the m-tiles [plan[tb], plan[te]), with the given
// block of eight claim counters.
template <class C>
hipError_t launch(const FfnArgs& a, int phase, hipStream_t s, int tb, int te, int ctr_block, int reserve) {
  const int wide = a.I > a.Is ? a.I : a.Is;
  const int ntn = phase == 1 ? (wide + C::BN / 2 - 1) / (C::BN / 2) : (a.H + C::BN - 1) / C::BN;
  const int grid = (cu_count() * C::WG_PER_CU + 7) / 8 * 8;  // resident workgroups, a multiple of 8 XCDs
  // Each XCD takes grid/8 consecutive tiles of a round: supertiles of 4
  // m-tiles, so an XCD's 28 or 32 tiles at a time are about 4 m-tiles x 7-8
  // n-tiles, each weight slice serving 4 m-tiles and each A slice 7-8 n-tiles
  // from L2.  On the 8192-token skewed layer 4 measured 1.6% faster than 8
  // (10.86-10.88 against 11.02-11.08 ms per step) and within noise of 2 and
  // 3; 1 and 16 were slower.  (Two m-tiles x all n-tiles per XCD, which
  // fetches each A slice once, measured slower too.)
  const int super = 4;
  int32_t* ctr = const_cast<int32_t*>(a.plan) + kPlanCounters + (ctr_block * 2 + phase - 1) * 8;
  reserve = reserve < grid - 8 ? reserve / 8 * 8 : 0;
  if (phase == 1) ffn_tiles_kernel<C, 1><<<grid, C::NT, 0, s>>>(a, ntn, super, tb, te, ctr, reserve);
  else ffn_tiles_kernel<C, 2><<<grid, C::NT, 0, s>>>(a, ntn, super, tb, te, ctr, reserve);
  return hipGetLastError();
}

}  // namespace

bool ffn_dma_supported(const FfnArgs& a) {
  constexpr int k = BigCfg::BK;
  if (a.Is != 0 && a.Is % k != 0) return false;
  // fp8: whole 128 x 128 scale blocks, at most 128 K blocks (the LDS scale table)
  if (a.fp8) return a.H % 128 == 0 && a.I % 128 == 0 && a.H <= 128 * 128 && a.I <= 128 * 128;
  return a.H % k == 0 && a.I % k == 0;
}

hipError_t launch_ffn_gemm_big(const FfnArgs& a, int phase, hipStream_t s, int reserve) {
  if (!a.fp8) return launch<BigCfg>(a, phase, s, kPlanStart, kPlanTiles, 0, reserve);
  // fp8 layers: the routed groups' tiles decode codes; the shared expert's
  // [plan[2], plan[0]) tiles are bf16
  hipError_t e = launch<BigCfg8>(a, phase, s, kPlanStart, kPlanRoutedTiles, 0, reserve);
  if (e == hipSuccess && a.Is > 0) e = launch<BigCfg>(a, phase, s, kPlanRoutedTiles, kPlanTiles, 1, reserve);
  return e;
}

}  // namespace moe
