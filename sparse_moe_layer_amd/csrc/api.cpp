// C ABI of the routed MoE layer: host-side validation, workspace carving and
// stream-ordered launches.  Declarations and the contract of every entry
// point are in include/moe_mi355x.h.
#include "moe_mi355x.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace {

using moe::FfnArgs;

constexpr size_t kAlign = 256;
inline size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(const moe_problem* p) { return p->act_dtype == MOE_F32 ? 4 : 2; }
size_t w_bytes(const moe_problem* p) {
  return p->w_dtype == MOE_F32 ? 4 : (p->w_dtype == MOE_BF16 ? 2 : 1);
}

// ---------------------------------------------------------------------------
// router form: fp32 SIMT (fp32 layers), split-K weight streaming (T <= 16, the
// router is a GEMV bound by reading W_r; K split so that ~128 K values fall to
// each wave), or split-K MFMA GEMM (larger T).
// The logits land as nsplit fp32 partials that the top-k kernel adds.
// ---------------------------------------------------------------------------
struct RoutePlan {
  bool stream;
  int nsplit;
};

RoutePlan route_plan(const moe_problem* p) {
  if (p->act_dtype == MOE_F32) return {false, 1};
  if (p->T <= moe::kStreamMaxRows) return {true, moe::router_stream_split((int)p->H)};
  return {false, moe::router_gemm_split((int)p->T, (int)p->H, (int)p->E)};
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct StageSizes {
  size_t route, dispatch, ffn, stage;  // scratch of each stage; stage = max
};

StageSizes stage_sizes(const moe_problem* p) {
  StageSizes s{};
  const size_t T = (size_t)p->T, E = (size_t)p->E, k = (size_t)p->k;
  const size_t R = T * k;
  s.route = up((size_t)route_plan(p).nsplit * T * (E + 1) * 4) + kAlign;  // partials, then one counter
  s.dispatch = up(moe::dispatch_ws_ints(p->T, p->E) * 4);
  s.ffn = up(moe::ffn_plan_ints(p->T, p->E, p->k, p->I_shared > 0) * 4) + up(R * (size_t)p->I * act_bytes(p)) +
          up(T * (size_t)p->I_shared * act_bytes(p));
  s.stage = s.route;
  if (s.dispatch > s.stage) s.stage = s.dispatch;
  if (s.ffn > s.stage) s.stage = s.ffn;
  return s;
}

struct LayerWs {
  int32_t* ids;
  float* w;
  float* sl;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* pos;
  void* y;
  void* y_sh;
  void* stage;
  size_t total;
};

LayerWs layer_layout(const moe_problem* p, void* base) {
  const size_t T = (size_t)p->T, E = (size_t)p->E, k = (size_t)p->k, H = (size_t)p->H;
  const size_t R = T * k;
  char* b = static_cast<char*>(base);
  size_t o = 0;
  LayerWs L{};
  auto take = [&](size_t bytes) {
    char* r = b ? b + o : nullptr;
    o += up(bytes);
    return r;
  };
  L.ids = reinterpret_cast<int32_t*>(take(R * 4));
  L.w = reinterpret_cast<float*>(take(R * 4));
  L.sl = reinterpret_cast<float*>(take(T * 4));
  L.offsets = reinterpret_cast<int32_t*>(take((E + 1) * 4));
  L.sorted = reinterpret_cast<int32_t*>(take(R * 4));
  L.pos = reinterpret_cast<int32_t*>(take(R * 4));
  L.y = take(R * H * act_bytes(p));
  L.y_sh = take(p->I_shared > 0 ? T * H * act_bytes(p) : 0);
  L.stage = take(stage_sizes(p).stage);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------
moe_status check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_NULL;
  if (p->T < 0 || p->H < 1 || p->E < 1 || p->E > moe::kMaxExperts || p->k < 1 || p->k > p->E || p->k > 64 || p->I < 1 ||
      p->I_shared < 0)
    return MOE_ERR_SHAPE;
  if (p->T > (int64_t)INT32_MAX / p->k || p->H > (1 << 24) || p->I > (1 << 24) || p->I_shared > (1 << 24))
    return MOE_ERR_SHAPE;
  // kernels address x, h, h_sh and one expert's matrices with 32-bit element
  // offsets (the tile kernel's buffer loads with 32-bit byte offsets of bf16
  // elements); y [R, H] rows go through 64-bit offsets
  const int64_t lim = (int64_t)1 << 31;
  const int64_t R = p->T * p->k;
  if (p->T * p->H >= lim || R * p->I >= lim || p->T * p->I_shared >= lim || p->I * p->H >= lim ||
      p->I_shared * p->H >= lim)
    return MOE_ERR_UNSUPPORTED;
  const bool f32 = p->act_dtype == MOE_F32 && p->w_dtype == MOE_F32;
  const bool bf = p->act_dtype == MOE_BF16 && p->w_dtype == MOE_BF16;
  const bool fp8 = p->act_dtype == MOE_BF16 && p->w_dtype == MOE_FP8_E4M3FN;
  if (!f32 && !bf && !fp8) return MOE_ERR_DTYPE;
  const int64_t q = f32 ? 4 : 8;  // 16-byte vectors along every K-contiguous row
  if (p->H % q || p->I % q || p->I_shared % q) return MOE_ERR_UNSUPPORTED;
  if (fp8 && (p->scale_block != 128 || p->H % 128 || p->I % 128)) return MOE_ERR_UNSUPPORTED;
  const uint32_t known = MOE_FLAG_FORCE_GEMM | MOE_FLAG_FORCE_STREAM | MOE_FLAG_GEMM_TILE_128 | MOE_FLAG_GEMM_TILE_256 |
                         MOE_FLAG_PAGE_ROUTING;
  if (p->flags & ~known) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_FORCE_GEMM) && (p->flags & MOE_FLAG_FORCE_STREAM)) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_GEMM_TILE_128) && (p->flags & MOE_FLAG_GEMM_TILE_256)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_ws(const moe_problem* p, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return MOE_ERR_ALIGN;
  if (ws_bytes < moe_workspace_bytes(p)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status check_weights(const moe_problem* p, const moe_weights* w, bool need_router, bool need_experts) {
  if (!w) return MOE_ERR_NULL;
  if (need_router && !w->w_router) return MOE_ERR_NULL;
  if (need_router && !al16(w->w_router)) return MOE_ERR_ALIGN;
  if (need_experts) {
    if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL;
    if (!al16(w->w_gate) || !al16(w->w_up) || !al16(w->w_down)) return MOE_ERR_ALIGN;
    if (w->stride_gate < 0 || w->stride_up < 0 || w->stride_down < 0) return MOE_ERR_SHAPE;
    const int64_t wb = (int64_t)w_bytes(p);
    if ((w->stride_gate * wb) % 16 || (w->stride_up * wb) % 16 || (w->stride_down * wb) % 16) return MOE_ERR_ALIGN;
    if (p->w_dtype == MOE_FP8_E4M3FN) {
      if (!w->s_gate || !w->s_up || !w->s_down) return MOE_ERR_NULL;
      if (!al16(w->s_gate) || !al16(w->s_up) || !al16(w->s_down)) return MOE_ERR_ALIGN;
    }
    if (p->I_shared > 0) {
      if (!w->sh_gate || !w->sh_up || !w->sh_down) return MOE_ERR_NULL;
      if (!al16(w->sh_gate) || !al16(w->sh_up) || !al16(w->sh_down)) return MOE_ERR_ALIGN;
    }
  }
  if (need_router && p->I_shared > 0) {
    if (!w->sh_gate_w) return MOE_ERR_NULL;
    if (!al16(w->sh_gate_w)) return MOE_ERR_ALIGN;
  }
  return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---------------------------------------------------------------------------
// stage bodies (arguments already validated)
// ---------------------------------------------------------------------------
// Where the layer call's small batches (T <= kSmallBatch) take the dispatch
// from the top-k kernel itself (fp32 layers, fp8 weights, or the GEMM path
// forced; bf16 layers take it in the gate/up streaming launch instead).  Such
// a batch always routes with the streaming (or fp32) router, whose launch
// zeroes the top-k counter.
static_assert(moe::kSmallBatch <= moe::kStreamMaxRows, "small batches take the streaming router");
struct DispatchOut {
  int32_t* offsets;
  int32_t* sorted;
  int32_t* pos;
};

moe_status do_route(const moe_problem* p, const void* x, const void* w_router, const void* sh_gate_w,
                    int32_t* ids, float* w, float* sl, void* stage, hipStream_t s,
                    const DispatchOut* d = nullptr) {
  const int T = (int)p->T, H = (int)p->H, E = (int)p->E, k = (int)p->k;
  const void* wsg = (sh_gate_w && sl) ? sh_gate_w : nullptr;
  float* partial = static_cast<float*>(stage);
  const RoutePlan rp = route_plan(p);
  // the fused small-batch top-k's counter, after the partial logits; the
  // router launch zeroes it
  const bool fused = d && T <= moe::kSmallBatch;
  int32_t* counter = reinterpret_cast<int32_t*>(static_cast<char*>(stage) +
                                                up((size_t)rp.nsplit * T * (E + 1) * 4));
  hipError_t e;
  if (p->act_dtype == MOE_F32)
    e = moe::launch_router_logits_f32(static_cast<const float*>(x), static_cast<const float*>(w_router),
                                      static_cast<const float*>(wsg), partial, T, H, E, s, fused ? counter : nullptr);
  else if (rp.stream)
    e = moe::launch_router_stream(x, w_router, wsg, partial, T, H, E, rp.nsplit, s, fused ? counter : nullptr);
  else
    e = moe::launch_router_logits_bf16(x, w_router, wsg, partial, T, H, E, rp.nsplit, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  const bool page = p->act_dtype == MOE_BF16 && (p->flags & MOE_FLAG_PAGE_ROUTING);
  if (fused)
    return hip_status(moe::launch_topk_dispatch_small(partial, rp.nsplit, E + (wsg ? 1 : 0), T, E, k, wsg ? 1 : 0,
                                                      page, ids, w, sl, d->offsets, d->sorted, d->pos, counter, s));
  return hip_status(moe::launch_topk(partial, rp.nsplit, E + (wsg ? 1 : 0), T, E, k, wsg ? 1 : 0, page, ids, w, sl, s));
}

FfnArgs ffn_args(const moe_problem* p, const moe_weights* w, const void* x, const int32_t* offsets,
                 const int32_t* sorted, bool shared) {
  FfnArgs a{};
  a.T = (int)p->T;
  a.H = (int)p->H;
  a.E = (int)p->E;
  a.k = (int)p->k;
  a.I = (int)p->I;
  a.Is = (p->I_shared > 0 && shared) ? (int)p->I_shared : 0;
  a.fp8 = p->w_dtype == MOE_FP8_E4M3FN;
  a.x = x;
  a.offsets = offsets;
  a.sorted = sorted;
  a.wg = w->w_gate;
  a.wu = w->w_up;
  a.wd = w->w_down;
  a.sg = w->stride_gate ? w->stride_gate : p->I * p->H;
  a.su = w->stride_up ? w->stride_up : p->I * p->H;
  a.sd = w->stride_down ? w->stride_down : p->H * p->I;
  a.scg = w->s_gate;
  a.scu = w->s_up;
  a.scd = w->s_down;
  a.shg = w->sh_gate;
  a.shu = w->sh_up;
  a.shd = w->sh_down;
  return a;
}

// Grouped GEMM path: the persistent direct-load kernel with 256-row tiles
// once experts average 128 rows or more (the MFMA rate bounds them), else
// the register-staged kernel with 128-row tiles (about a hundred rows per
// expert: weight streaming bounds them).  The 256-row tiles take H, I and
// I_shared multiples of 32.  The caller can pin either tiling for A/B runs.
bool use_big_tiles(const moe_problem* p, const FfnArgs& a) {
  if (!moe::ffn_dma_supported(a)) return false;
  if (p->flags & MOE_FLAG_GEMM_TILE_128) return false;
  if (p->flags & MOE_FLAG_GEMM_TILE_256) return true;
  // bf16 weights: once experts average 128 rows.  fp8 weights: from 32 rows
  // (the 128-row fp8 tiles decode every weight once per m-tile; on the
  // skewed 2.4T layer at 40 rows per expert the 256-row tiles of its large
  // groups measured faster).
  return p->T * p->k >= (a.fp8 ? 32 : 128) * p->E;
}

// A second stream per device (default priority) and two events, so that
// the MFMA-bound tile launches and the HBM-bound streaming launches of one
// FFN call run side by side: fork after the plan kernel, join before the
// call returns.  Created on first use; a device where that fails runs the
// launches in order on the caller's stream.  The mutex keeps each fork's
// record/wait pairs and the launches between them from interleaving with
// another host thread's.
struct Aux {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};
constexpr int kMaxDevices = 64;
Aux g_aux[kMaxDevices];
std::mutex g_aux_init;

Aux* aux_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_aux_init);
  Aux& x = g_aux[dev];
  if (!x.s2) {
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    x.fork = a;
    x.join = b;
    x.s2 = st;
  }
  return &x;
}

// Workgroups of the persistent tile grid left to a streaming launch that
// runs beside it (4 per XCD): the tiles are partly bound by the chip's
// power, so they lose less than the CUs' share, and the streams' HBM reads
// overlap them.
constexpr int kStreamReserve = 32;

// phases: bit 0 gate/up, bit 1 down.  The plan kernel runs first (bf16/fp8).
// fork_ok: the streaming launches may run on the device's second stream.
// route (may be null): the gate/up streaming launch takes the small batch's
// dispatch from the ids (see moe::SmallRoute).
moe_status run_ffn(const moe_problem* p, FfnArgs& a, int phases, void* plan_ws, hipStream_t s, bool fork_ok,
                   const moe::SmallRoute* route = nullptr) {
  if (p->act_dtype == MOE_F32) return hip_status(moe::launch_ffn_f32(a, phases, s));
  int32_t* plan = static_cast<int32_t*>(plan_ws);
  const bool big = use_big_tiles(p, a);
  // Groups of at most kStreamMaxRows rows stream their weights after the
  // tiles.  (As ragged 256-row tiles they measured slower: the 2.4T fp8
  // layer 4.26 against 3.75 ms per step.)
  const int stream_rows = moe::kStreamMaxRows;
  // A group holds at most T rows, so with T <= stream_rows no group can
  // reach the GEMM path unless it is forced; with the GEMM path forced no
  // group streams.  Launches that cannot have work are skipped.
  const bool any_gemm = (p->flags & MOE_FLAG_FORCE_GEMM) ||
                        (!(p->flags & MOE_FLAG_FORCE_STREAM) && p->T > stream_rows);
  const bool any_stream = !(p->flags & MOE_FLAG_FORCE_GEMM);
  // Every group streaming as one m-block (T <= kStreamMaxRows): the
  // streaming kernels list the groups themselves, with no plan kernel ahead
  // of them in the chain.
  const bool self_plan = !any_gemm && p->T <= moe::kStreamMaxRows;
  if (!self_plan) {
    if (moe::launch_ffn_plan(a.offsets, a.sorted, a.T, a.E, a.k, a.Is > 0 ? 1 : 0, p->flags,
                             big ? moe::kGemmBigBM : moe::kGemmBM, stream_rows, plan, s) != hipSuccess)
      return MOE_ERR_HIP;
    moe::ffn_bind_plan(a, plan);
  }
  // the 256-row tiles and the streaming groups side by side
  Aux* x = (fork_ok && big && any_gemm && any_stream && !self_plan) ? aux_stream() : nullptr;
  if (!x) {
    for (int phase = 1; phase <= 2; ++phase) {
      if (!(phases & phase)) continue;
      if (any_gemm) {
        const hipError_t e = big ? moe::launch_ffn_gemm_big(a, phase, s) : moe::launch_ffn_gemm(a, phase, s);
        if (e != hipSuccess) return MOE_ERR_HIP;
      }
      if (any_stream &&
          moe::launch_ffn_stream(a, phase, s, self_plan, phase == 1 ? route : nullptr) != hipSuccess)
        return MOE_ERR_HIP;
    }
    return MOE_OK;
  }
  std::lock_guard<std::mutex> lk(x->mu);
  if (hipEventRecord(x->fork, s) != hipSuccess || hipStreamWaitEvent(x->s2, x->fork, 0) != hipSuccess)
    return MOE_ERR_HIP;
  moe_status st = MOE_OK;
  for (int phase = 1; phase <= 2 && st == MOE_OK; ++phase) {
    if (!(phases & phase)) continue;
    if (moe::launch_ffn_gemm_big(a, phase, s, kStreamReserve) != hipSuccess ||
        moe::launch_ffn_stream(a, phase, x->s2, false) != hipSuccess)
      st = MOE_ERR_HIP;
  }
  // the join is recorded even after a failed launch, so the caller's stream
  // never runs ahead of the second stream's work
  if (hipEventRecord(x->join, x->s2) != hipSuccess || hipStreamWaitEvent(s, x->join, 0) != hipSuccess)
    return MOE_ERR_HIP;
  return st;
}

moe_status do_ffn(const moe_problem* p, const moe_weights* w, const void* x, const int32_t* offsets,
                  const int32_t* sorted, void* y, void* y_sh, void* stage, hipStream_t s, bool fork_ok = true,
                  const moe::SmallRoute* route = nullptr) {
  FfnArgs a = ffn_args(p, w, x, offsets, sorted, y_sh != nullptr);
  a.y = y;
  a.y_sh = a.Is ? y_sh : nullptr;
  // stage scratch: plan ints | h | h_sh
  char* b = static_cast<char*>(stage);
  const size_t plan_bytes = up(moe::ffn_plan_ints(p->T, p->E, p->k, a.Is > 0) * 4);
  a.h = b + plan_bytes;
  a.h_sh = b + plan_bytes + up((size_t)p->T * p->k * p->I * act_bytes(p));
  return run_ffn(p, a, 3, b, s, fork_ok, route);
}

}  // namespace

namespace moe {

moe_status layer_forward_checks(const moe_problem* p, const moe_weights* w, const void* x, const void* out) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if ((st = check_weights(p, w, true, true)) != MOE_OK) return st;
  if (!x || !out) return MOE_ERR_NULL;
  if (!al16(x) || !al16(out)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status layer_forward_run(const moe_problem* p, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_ids, float* topk_w, void* ws, hipStream_t s, bool fork_ok) {
  moe_status st;
  LayerWs L = layer_layout(p, ws);
  int32_t* ids = topk_ids ? topk_ids : L.ids;
  float* tw = topk_w ? topk_w : L.w;
  const bool sh = p->I_shared > 0;
  // A small batch's dispatch comes out of the gate/up streaming launch (bf16
  // weights, every group streaming) or else out of the top-k workgroups; a
  // larger batch's from the dispatch kernels.
  const bool small = p->T <= moe::kSmallBatch;
  const bool route_in_ffn = small && p->act_dtype == MOE_BF16 && p->w_dtype == MOE_BF16 &&
                            !(p->flags & MOE_FLAG_FORCE_GEMM);
  const DispatchOut d{L.offsets, L.sorted, L.pos};
  const moe::SmallRoute route{ids, L.offsets, L.sorted, L.pos};
  if ((st = do_route(p, x, w->w_router, sh ? w->sh_gate_w : nullptr, ids, tw, sh ? L.sl : nullptr, L.stage, s,
                     small && !route_in_ffn ? &d : nullptr)) != MOE_OK)
    return st;
  if (!small && (st = hip_status(moe::launch_dispatch(ids, (int)p->T, (int)p->E, (int)p->k, L.offsets, L.sorted,
                                                      L.pos, static_cast<int32_t*>(L.stage), s,
                                                      /*distinct=*/true))) != MOE_OK)
    return st;
  if ((st = do_ffn(p, w, x, L.offsets, L.sorted, L.y, sh ? L.y_sh : nullptr, L.stage, s, fork_ok,
                   route_in_ffn ? &route : nullptr)) != MOE_OK)
    return st;
  return hip_status(moe::launch_combine(L.y, L.pos, tw, sh ? L.y_sh : nullptr, sh ? L.sl : nullptr, out, (int)p->T,
                                        (int)p->H, (int)p->k, p->act_dtype == MOE_F32 ? 1 : 0, s));
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range";
    case MOE_ERR_DTYPE: return "unsupported dtype combination";
    case MOE_ERR_ALIGN: return "misaligned pointer or stride";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "shape or flags not supported by the kernels";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_validate(const moe_problem* p) { return check_problem(p); }

size_t moe_workspace_bytes(const moe_problem* p) {
  if (check_problem(p) != MOE_OK) return 0;
  return layer_layout(p, nullptr).total;
}

moe_status moe_route(const moe_problem* p, const void* x, const void* w_router, const void* sh_gate_w,
                     int32_t* topk_ids, float* topk_w, float* shared_logit, void* ws, size_t ws_bytes,
                     void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_NULL;
  if (!al16(x) || !al16(w_router) || (sh_gate_w && !al16(sh_gate_w))) return MOE_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  return do_route(p, x, w_router, sh_gate_w, topk_ids, topk_w, shared_logit, ws, (hipStream_t)stream);
}

moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_ids, int32_t* expert_offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if (!topk_ids || !expert_offsets || !sorted_assign || !assign_pos) return MOE_ERR_NULL;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_dispatch(topk_ids, (int)p->T, (int)p->E, (int)p->k, expert_offsets, sorted_assign,
                                         assign_pos, static_cast<int32_t*>(ws), (hipStream_t)stream));
}

moe_status moe_expert_ffn(const moe_problem* p, const moe_weights* w, const void* x, const int32_t* expert_offsets,
                          const int32_t* sorted_assign, void* y, void* y_shared, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if ((st = check_weights(p, w, false, true)) != MOE_OK) return st;
  if (!x || !expert_offsets || !sorted_assign || !y) return MOE_ERR_NULL;
  if (!al16(x) || !al16(y) || (y_shared && !al16(y_shared))) return MOE_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  return do_ffn(p, w, x, expert_offsets, sorted_assign, y, y_shared, ws, (hipStream_t)stream);
}

moe_status moe_expert_gate_up(const moe_problem* p, const moe_weights* w, const void* x,
                              const int32_t* expert_offsets, const int32_t* sorted_assign, void* h, void* h_shared,
                              void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if ((st = check_weights(p, w, false, true)) != MOE_OK) return st;
  if (!x || !expert_offsets || !sorted_assign || !h) return MOE_ERR_NULL;
  if (!al16(x) || !al16(h) || (h_shared && !al16(h_shared))) return MOE_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  FfnArgs a = ffn_args(p, w, x, expert_offsets, sorted_assign, h_shared != nullptr);
  a.h = h;
  a.h_sh = a.Is ? h_shared : nullptr;
  return run_ffn(p, a, 1, ws, (hipStream_t)stream, true);
}

moe_status moe_expert_down(const moe_problem* p, const moe_weights* w, const int32_t* expert_offsets,
                           const void* h, const void* h_shared, void* y, void* y_shared, void* ws, size_t ws_bytes,
                           void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if ((st = check_weights(p, w, false, true)) != MOE_OK) return st;
  if (!expert_offsets || !h || !y) return MOE_ERR_NULL;
  if ((h_shared == nullptr) != (y_shared == nullptr)) return MOE_ERR_NULL;
  if (!al16(h) || !al16(y) || (h_shared && !al16(h_shared)) || (y_shared && !al16(y_shared))) return MOE_ERR_ALIGN;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  FfnArgs a = ffn_args(p, w, nullptr, expert_offsets, nullptr, y_shared != nullptr);
  a.h = const_cast<void*>(h);
  a.h_sh = a.Is ? const_cast<void*>(h_shared) : nullptr;
  a.y = y;
  a.y_sh = a.Is ? y_shared : nullptr;
  return run_ffn(p, a, 2, ws, (hipStream_t)stream, true);
}

moe_status moe_combine(const moe_problem* p, const void* y, const int32_t* assign_pos, const float* topk_w,
                       const void* y_shared, const float* shared_logit, void* out, void* stream) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // empty batch: nothing to read or write
  if (!y || !assign_pos || !topk_w || !out) return MOE_ERR_NULL;
  if ((y_shared == nullptr) != (shared_logit == nullptr)) return MOE_ERR_NULL;
  if (!al16(y) || !al16(out) || (y_shared && !al16(y_shared))) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(y, assign_pos, topk_w, y_shared, shared_logit, out, (int)p->T, (int)p->H,
                                        (int)p->k, p->act_dtype == MOE_F32 ? 1 : 0, (hipStream_t)stream));
}

moe_status moe_layer_forward(const moe_problem* p, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = moe::layer_forward_checks(p, w, x, out);
  if (st != MOE_OK || p->T == 0) return st;
  if ((st = check_ws(p, ws, ws_bytes)) != MOE_OK) return st;
  return moe::layer_forward_run(p, w, x, out, topk_ids, topk_w, ws, (hipStream_t)stream);
}


// ---------------------------------------------------------------------------
// gated residual
// ---------------------------------------------------------------------------
static moe_status check_gr(const moe_problem* p, int64_t rank) {
  moe_status st = check_problem(p);
  if (st != MOE_OK) return st;
  if (p->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (p->H % 32 || rank < 16 || rank % 16 || rank > (1 << 16)) return MOE_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if (p->T * 4 * p->H >= lim || (rank + 4) * 4 * p->H >= lim || p->T * (rank + 4) >= lim) return MOE_ERR_SHAPE;
  return MOE_OK;
}

size_t moe_gr_workspace_bytes(const moe_problem* p, int64_t rank) {
  if (check_gr(p, rank) != MOE_OK) return 0;
  return moe::gr_workspace_bytes(p->T, p->H, rank);
}

moe_status moe_gr_read(const moe_problem* p, const moe_gr_weights* g, const void* resid, void* x, float* s,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!p || !g) return MOE_ERR_NULL;
  moe_status st = check_gr(p, g->rank);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!g->norm_w || !g->w_read || !g->w_up || !resid || !x || !s || !ws) return MOE_ERR_NULL;
  if (!al16(g->norm_w) || !al16(g->w_read) || !al16(g->w_up) || !al16(resid) || !al16(x) || !al16(s) ||
      reinterpret_cast<uintptr_t>(ws) % kAlign)
    return MOE_ERR_ALIGN;
  if (ws_bytes < moe::gr_workspace_bytes(p->T, p->H, g->rank)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_gr_read(resid, g->norm_w, g->w_read, g->w_up, g->eps, (int)p->T, (int)p->H,
                                        (int)g->rank, x, s, ws, (hipStream_t)stream));
}

moe_status moe_gr_write(const moe_problem* p, const void* resid, const float* s, const void* f, void* resid_out,
                        void* stream) {
  if (!p) return MOE_ERR_NULL;
  moe_status st = check_gr(p, 16);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!resid || !s || !f || !resid_out) return MOE_ERR_NULL;
  if (!al16(resid) || !al16(f) || !al16(resid_out) || reinterpret_cast<uintptr_t>(s) % 4) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_gr_write(resid, s, f, resid_out, (int)p->T, (int)p->H, (hipStream_t)stream));
}

moe_status moe_combine_gr_write(const moe_problem* p, const void* y, const int32_t* assign_pos,
                                const float* topk_w, const void* y_shared, const float* shared_logit,
                                const void* resid, const float* s, void* out, void* resid_out, void* stream) {
  if (!p) return MOE_ERR_NULL;
  moe_status st = check_gr(p, 16);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!y || !assign_pos || !topk_w || !resid || !s || !resid_out) return MOE_ERR_NULL;
  if ((y_shared == nullptr) != (shared_logit == nullptr)) return MOE_ERR_NULL;
  if (!al16(y) || !al16(resid) || !al16(resid_out) || (out && !al16(out)) || (y_shared && !al16(y_shared)) ||
      reinterpret_cast<uintptr_t>(s) % 4)
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine_gr_write(y, assign_pos, topk_w, y_shared, shared_logit, out, resid, s,
                                                 resid_out, (int)p->T, (int)p->H, (int)p->k, (hipStream_t)stream));
}

size_t moe_audit_workspace_bytes(int64_t slices) {
  if (slices < 1 || slices > 65535) return 0;
  return moe::audit_workspace_bytes(slices);
}

moe_status moe_weight_audit(const void* w, int32_t dtype, int64_t slices, int64_t n, int64_t slice_stride,
                            moe_audit_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (slices < 1 || slices > 65535 || n < 0 || n >= ((int64_t)1 << 32) || slice_stride < n) return MOE_ERR_SHAPE;
  if ((n > 0 && !w) || !stats || !ws) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(w) & 1u) || (reinterpret_cast<uintptr_t>(stats) & 7u) ||
      reinterpret_cast<uintptr_t>(ws) % kAlign)
    return MOE_ERR_ALIGN;
  if (ws_bytes < moe::audit_workspace_bytes(slices)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_audit(w, slices, n, slice_stride, stats, ws, (hipStream_t)stream));
}

}  // extern "C"
