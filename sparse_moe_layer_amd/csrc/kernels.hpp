// Host-visible launchers of the MoE kernels.  Every launcher enqueues on
// `stream` and returns hipGetLastError() of its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_mi355x.h"

namespace moe {

// Rows per MFMA GEMM m-tile (128-row kernels / big-tile kernel) and per
// streaming m-block.
constexpr int kGemmBM = 128;
constexpr int kGemmBigBM = 256;
constexpr int kStreamBM = 16;
constexpr int kMaxExperts = 1024;
// Batches of at most this many tokens route and dispatch in one workgroup
// (a wave per token).
constexpr int kSmallBatch = 16;
// plan ints ahead of the work lists: [0] m-tiles, [1] stream m-blocks,
// [2] / [3] where the shared expert's m-tiles / m-blocks begin, then the
// fused kernel's claim counters: kPlanCounters + (launch * 2 + phase - 1) * 8,
// eight per XCD-indexed counter block, zeroed by the plan kernel
constexpr int kPlanCounters = 8;
constexpr int kPlanHeader = kPlanCounters + 4 * 8;
// Positions in the plan header, as the kernels' list bounds: a kernel runs
// the entries [plan[begin], plan[end]) of its list, begin kPlanStart meaning 0.
enum PlanPos : int {
  kPlanStart = -1,
  kPlanTiles = 0,          // end of the m-tile list
  kPlanBlocks = 1,         // end of the stream m-block list
  kPlanRoutedTiles = 2,    // end of the routed groups' m-tiles (the shared expert's follow)
  kPlanRoutedBlocks = 3,   // end of the routed groups' m-blocks (the shared expert's follow)
};
// An expert with at most this many rows streams its weights (small-M path).
constexpr int kStreamMaxRows = 16;

// Everything the grouped expert kernels need to resolve a group (routed
// expert g < E, or the shared expert g == E) and its operands.
struct FfnArgs {
  int T, H, E, k, I, Is;
  int fp8;                    // routed weights are e4m3fn codes + fp32 block scales
  const void* x;              // [T, H] bf16
  const int32_t* offsets;     // [E+1]
  const int32_t* sorted;      // [R]
  const void* wg; const void* wu; const void* wd;  // routed, elements: bf16 or u8 codes
  int64_t sg, su, sd;         // expert strides (elements)
  const float* scg; const float* scu; const float* scd;  // fp8 block scales
  const void* shg; const void* shu; const void* shd;     // shared expert (bf16) or null
  void* h;                    // [R, I]  bf16 hidden of routed rows
  void* h_sh;                 // [T, Is] bf16 hidden of the shared expert
  void* y;                    // [R, H]  bf16
  void* y_sh;                 // [T, H]  bf16 (may be null when Is == 0)
  // device-built work lists
  const int32_t* plan;        // kPlanHeader ints (see there), then the lists
  const int32_t* mt_group; const int32_t* mt_row0;
  const int32_t* sb_group; const int32_t* sb_row0;
  const int32_t* sb_base;   // first dispatched row of the group (0 for the shared expert)
  const int32_t* sb_nrows;  // rows of the m-block (<= kStreamBM)
  const int32_t* sb_tok;    // [sb][kStreamBM] token of each row (gate/up gather)
};

size_t ffn_plan_ints(int64_t T, int64_t E, int64_t k, bool shared);

// Router logits as nsplit fp32 partial sums over K chunks: partial[c][t][n],
// n < E router rows, n == E the shared gate (when w_sg != null).  The top-k
// kernel adds the chunks in order c = 0..nsplit-1.  The small-batch
// streaming router writes complete logits (nsplit = 1).
// max_split: the largest split taken when it needs more than one round.
int router_gemm_split(int T, int H, int E, int max_split = 4);
// gated_residual: the same GEMM for the gated residual's read projection
// (a separately named kernel instance, so traces tell the two apart).
hipError_t launch_router_logits_bf16(const void* x, const void* w_router, const void* w_sg,
                                     float* partial, int T, int H, int E, int nsplit, hipStream_t s,
                                     bool gated_residual = false);
// nsplit = router_stream_split(H) K chunks, each its own partial logits.
int router_stream_split(int H);
// zero_word (may be null): an int the launch sets to zero for the kernel
// that follows it (the small-batch top-k counter).
hipError_t launch_router_stream(const void* x, const void* w_router, const void* w_sg, float* logits, int T,
                                int H, int E, int nsplit, hipStream_t s, int32_t* zero_word = nullptr);
hipError_t launch_router_logits_f32(const float* x, const float* w_router, const float* w_sg,
                                    float* logits, int T, int H, int E, hipStream_t s,
                                    int32_t* zero_word = nullptr);
// page: round the logits to bf16 before the top-k and the mixing weights to
// bf16 after renormalising (the page's routing numerics for bf16 layers).
hipError_t launch_topk(const float* partial, int nsplit, int ldl, int T, int E, int k, int has_sg, bool page,
                       int32_t* ids, float* w, float* shared_logit, hipStream_t s);
size_t dispatch_ws_ints(int64_t T, int64_t E);
// distinct: the ids come from the router, which never repeats an expert
// within a token (skips the per-token check for repeats).
// Top-k and dispatch in one kernel for 1 <= T <= kSmallBatch (same outputs
// as launch_topk followed by launch_dispatch).  counter: one int, zero at
// launch (the router launch zeroes it), left at zero.
hipError_t launch_topk_dispatch_small(const float* partial, int nsplit, int ldl, int T, int E, int k, int has_sg,
                                     bool page, int32_t* ids, float* w, float* shared_logit, int32_t* offsets,
                                     int32_t* sorted, int32_t* pos, int32_t* counter, hipStream_t s);
hipError_t launch_dispatch(const int32_t* ids, int T, int E, int k, int32_t* offsets,
                           int32_t* sorted, int32_t* pos, int32_t* ws, hipStream_t s, bool distinct = false);
// Groups of more than stream_rows rows (and none with MOE_FLAG_FORCE_STREAM,
// all with MOE_FLAG_FORCE_GEMM) become m-tiles of bm rows, the rest 16-row
// streaming m-blocks.
hipError_t launch_ffn_plan(const int32_t* offsets, const int32_t* sorted, int T, int E, int k, int has_shared,
                           uint32_t flags, int bm, int stream_rows, int32_t* plan_ws, hipStream_t s);
void ffn_bind_plan(FfnArgs& a, int32_t* plan_ws);
// phase 1 gate/up, 2 down: the 128-row MFMA tiles over the m-tile list
hipError_t launch_ffn_gemm(const FfnArgs& a, int phase, hipStream_t s);
// Persistent direct-load MFMA GEMM with 256-row tiles for layers with
// hundreds of rows per expert (ragged last m-tiles included; bf16 weights
// need H, I and I_shared multiples of 32).
bool ffn_dma_supported(const FfnArgs& a);
// reserve: workgroups of the persistent grid that leave at once when the
// plan has streaming blocks, so that a streaming launch on another stream
// gets their CUs (0: the whole grid takes tiles).
hipError_t launch_ffn_gemm_big(const FfnArgs& a, int phase, hipStream_t s, int reserve = 0);
// A small batch's dispatch done by the gate/up streaming launch itself (bf16
// weights, T <= kSmallBatch): from the router's picks ids [T, k] (distinct
// within a token), every workgroup builds each expert's token mask and the
// list of touched experts in LDS, and workgroup 0 writes offsets [E+1],
// sorted [R] and pos [R] (the outputs of launch_dispatch) for the launches
// after it.
struct SmallRoute {
  const int32_t* ids;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* pos;
};
// phase 1 gate/up, 2 down.  self_plan: T <= kStreamMaxRows and no plan kernel
// ran; the kernels list the touched groups from the offsets themselves, or
// (route, phase 1 with bf16 weights and T <= kSmallBatch) from the ids.
hipError_t launch_ffn_stream(const FfnArgs& a, int phase, hipStream_t s, bool self_plan = false,
                             const SmallRoute* route = nullptr);
hipError_t launch_ffn_f32(const FfnArgs& a, int phases, hipStream_t s);  // bit 0 gate/up, bit 1 down
hipError_t launch_combine(const void* y, const int32_t* pos, const float* w, const void* y_sh,
                          const float* shared_logit, void* out, int T, int H, int k, int f32,
                          hipStream_t s);
// bf16 combine with the gated-residual stream write in its epilogue: out
// (F(x), may be null) and resid_out [T, 4, H] = resid + gate[:, i] * F(x).
hipError_t launch_combine_gr_write(const void* y, const int32_t* pos, const float* w, const void* y_sh,
                                   const float* shared_logit, void* out, const void* resid, const float* gate,
                                   void* resid_out, int T, int H, int k, hipStream_t s);

// The whole layer behind moe_layer_forward: argument checks (MOE_OK also
// for an empty batch, which needs no run), then the launches on workspace
// ws of moe_workspace_bytes(p) bytes (no workspace check).  fork_ok: the
// FFN's streaming launches may run on the device's second stream (created
// on first use); false keeps every launch on s.
moe_status layer_forward_checks(const moe_problem* p, const moe_weights* w, const void* x, const void* out);
moe_status layer_forward_run(const moe_problem* p, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_ids, float* topk_w, void* ws, hipStream_t s, bool fork_ok = true);

// Gated residual read / write (bf16).
// Expert-weight audit (bf16): histograms of the bit patterns per slice and
// over the tensor, then the exact statistics of each.
size_t audit_workspace_bytes(int64_t slices);
hipError_t launch_audit(const void* w, int64_t slices, int64_t n, int64_t stride, moe_audit_stats* stats, void* ws,
                        hipStream_t st);
size_t gr_workspace_bytes(int64_t T, int64_t H, int64_t rank);
hipError_t launch_gr_read(const void* resid, const void* norm_w, const void* w_read, const void* w_up, float eps,
                          int T, int H, int rank, void* x, float* s, void* ws, hipStream_t st);
hipError_t launch_gr_write(const void* resid, const float* s, const void* f, void* out, int T, int H, hipStream_t st);

}  // namespace moe
