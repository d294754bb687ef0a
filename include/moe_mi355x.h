/*
 * moe_mi355x.h -- C ABI of the routed Mixture-of-Experts FFN layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (Qwen3.8-Flash-Next study, section "MoE: 512 experts behind a
 * width-640 intermediate", eq. expert(x) and eq. MoE(x)):
 *
 *   expert_e(x) = W_down[e] ( SiLU(W_gate[e] x) * (W_up[e] x) )
 *   out_t       = sum_{j<k} w[t,j] expert_{ids[t,j]}(x_t)
 *                 + sigmoid(w_sg . x_t) * shared(x_t)
 *
 * computed in the five stages of that section's pipeline figure: router
 * logits over the E experts, the k best per token with their weights
 * rescaled to sum to one, dispatch of the R = k*T (token, expert) pairs into
 * per-expert groups, the grouped expert products, and the weighted combine
 * with the gated shared expert.
 * One entry point per stage, plus the whole layer in one call.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers are device pointers (hipMalloc'd or equivalent) owned by the
 *    caller; the library never allocates or frees device memory for them and
 *    never synchronises.  Tensors are row-major and contiguous, except routed
 *    expert matrices, which may sit at any element stride from one expert to
 *    the next (moe_weights).
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued asynchronously and ordered after earlier work on it; no
 *    host<->device copy happens inside a call.  When an expert FFN call has
 *    both 256-row GEMM tiles and streamed groups, the streamed groups run on
 *    a second stream of the library's (one per device, default priority,
 *    created with two events on the first such call): forked from `stream`
 *    after the call's first kernel and joined back into it before the call's
 *    later work, so to the caller every call is ordered on `stream` alone
 *    (also under graph capture, where the fork and join become graph edges).
 *    Host threads that share a device serialise on that second stream's
 *    enqueue; a thread must not capture a graph while another uses the
 *    library on the same device.  moe_layer_forward_noalloc never forks.
 *  - `ws`/`ws_bytes` is caller-owned scratch device memory of at least
 *    moe_workspace_bytes(p) bytes, 256-byte aligned.  Its contents on entry
 *    do not matter; it must not be used by anything else until the stream has
 *    run the call.  Concurrent calls need distinct workspaces.
 *  - Validation happens on the host before any launch: a non-OK status means
 *    nothing was enqueued.  MOE_ERR_HIP reports a failed launch
 *    (hipGetLastError); faults during execution surface at the caller's next
 *    synchronisation.  NaN/Inf inputs give unspecified outputs.
 *  - T == 0 is a valid no-op returning MOE_OK once the problem itself is
 *    valid; no pointer is read or written (they may be NULL).
 *  - Routing ties: experts are ordered by descending fp32 logit, equal logits
 *    by ascending expert id.  Results are deterministic run to run.
 *  - Expert ids, the dispatch permutation and all integer outputs are exact;
 *    floating outputs carry fp32 accumulation and bf16 rounding of the
 *    intermediates h (the SwiGLU hidden) and y (per-assignment outputs).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                        */
  MOE_ERR_SHAPE = 2,       /* a size is out of range (T<0, k<1, k>E, E>1024, ...) */
  MOE_ERR_DTYPE = 3,       /* unsupported activation / weight dtype pair        */
  MOE_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned, or ws not 256   */
  MOE_ERR_WORKSPACE = 5,   /* ws_bytes < moe_workspace_bytes(p)                 */
  MOE_ERR_UNSUPPORTED = 6, /* valid shape the kernels do not cover (see below)  */
  MOE_ERR_HIP = 7          /* a kernel launch failed                            */
} moe_status;

typedef enum {
  MOE_F32 = 0,             /* IEEE binary32                                     */
  MOE_BF16 = 1,            /* bfloat16                                          */
  MOE_FP8_E4M3FN = 2       /* OCP E4M3FN codes (uint8) with fp32 block scales   */
} moe_dtype;

/* Problem description.  Supported combinations:
 *   act_dtype F32  with w_dtype F32   (all tensors fp32)
 *   act_dtype BF16 with w_dtype BF16
 *   act_dtype BF16 with w_dtype FP8_E4M3FN (routed experts only; router,
 *       shared expert and shared gate stay bf16 -- "Qwen3.8, weights in hand",
 *       section "What FP8 actually quantizes"); scale_block must be 128 and
 *       H, I multiples of 128.
 * Limits: 1 <= E <= 1024, 1 <= k <= min(E, 64), H and I multiples of 8 (bf16)
 * or of 4 (f32), I_shared 0 or a multiple of 8; T*k < 2^31; the tensors the
 * kernels address with 32-bit element offsets below 2^31 elements (T*H,
 * T*k*I, T*I_shared, I*H, I_shared*H).  The per-assignment outputs y [T*k, H]
 * are addressed with 64-bit offsets and may exceed 2^31 elements (e.g. a
 * 32768-token chunk of the 2.4T shape).                                       */
typedef struct {
  int64_t T;          /* tokens                                               */
  int64_t H;          /* hidden width                                          */
  int64_t E;          /* routed experts                                        */
  int64_t k;          /* experts chosen per token                              */
  int64_t I;          /* routed expert intermediate width                      */
  int64_t I_shared;   /* shared expert intermediate width; 0 = no shared expert */
  int32_t act_dtype;  /* moe_dtype of x, router, shared expert, y, out         */
  int32_t w_dtype;    /* moe_dtype of routed expert matrices                   */
  int32_t scale_block;/* fp8 scale block edge (128), else ignored              */
  uint32_t flags;     /* MOE_FLAG_* (0 = default)                              */
} moe_problem;

/* Force every routed expert onto the tiled MFMA GEMM path / the weight
 * streaming path (default: per expert, by its token count).  For A/B tests. */
#define MOE_FLAG_FORCE_GEMM   (1u << 0)
#define MOE_FLAG_FORCE_STREAM (1u << 1)
/* Tile height of the MFMA GEMM path: 128-row LDS-tiled kernel, or 256-row
 * direct-load kernel with each group's last m-tile of at most 128 rows in
 * the 128-row kernel (default: 256 when experts average >= 128 rows with
 * bf16 weights, >= 32 rows with fp8 weights).  The 256-row kernel needs
 * H, I, I_shared multiples of 32, and with fp8 weights H, I <= 16384;
 * otherwise the 128-row kernel runs whatever the flag says.  For A/B tests. */
#define MOE_FLAG_GEMM_TILE_128 (1u << 2)
#define MOE_FLAG_GEMM_TILE_256 (1u << 3)
/* Routing numerics of the Qwen3.8-Flash-Next study, MoE section, for bf16
 * layers: the softmax and top-k run on the router logits rounded to bf16
 * (equal rounded logits go to the lower expert id), and the renormalised
 * mixing weights are rounded to bf16 (returned in the fp32 topk_w).  Without
 * the flag the logits and weights stay fp32.  No effect on fp32 layers (their
 * activation dtype is fp32) or on the shared expert's gate logit. */
#define MOE_FLAG_PAGE_ROUTING (1u << 4)

/* Weights.  Layouts follow PyTorch Linear (out x in), which matches the GGUF
 * shapes on the Qwen3.8-2.4T-A95B hub discussion's zero-fraction table
 * (ffn_gate_exps 8192x2048x512 innermost-first = [E][I][H] row-major):
 *   w_router  [E, H]     act dtype
 *   w_gate    [E][I, H]  w_dtype, expert e at w_gate + e*stride_gate elements
 *   w_up      [E][I, H]  w_dtype, expert e at w_up   + e*stride_up
 *   w_down    [E][H, I]  w_dtype, expert e at w_down + e*stride_down
 *             stride 0 means dense (I*H).  A fused [E, 2I, H] gate_up tensor
 *             is passed as w_gate = base, w_up = base + I*H, strides 2*I*H.
 *   s_gate/s_up [E, I/128, H/128] fp32, s_down [E, H/128, I/128] fp32:
 *             fp8 block scales (value = code * scale); NULL unless fp8.
 *   sh_gate, sh_up [I_shared, H], sh_down [H, I_shared], sh_gate_w [1, H]:
 *             shared expert and its gate projection, act dtype; NULL iff
 *             I_shared == 0.                                                 */
typedef struct {
  const void* w_router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  int64_t stride_gate;
  int64_t stride_up;
  int64_t stride_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
  const void* sh_gate_w;
} moe_weights;

/* ABI version (MOE_ABI_VERSION) and a static string for a status code. */
int moe_abi_version(void);
const char* moe_status_str(moe_status s);

/* Host-only check of a problem description (no device access).  Returns the
 * status every entry point would return for these sizes and dtypes. */
moe_status moe_validate(const moe_problem* p);

/* Bytes of workspace every entry point below needs for problem p (the
 * maximum over entry points; 0 if p is invalid).  Host only. */
size_t moe_workspace_bytes(const moe_problem* p);

/* Router, softmax, top-k and renormalisation (the router and top-k stages of
 * the pipeline figure in the Qwen3.8-Flash-Next study's MoE section, which
 * renormalises the chosen experts' probabilities to sum to one).
 *   x [T,H] act, w_router [E,H] act, sh_gate_w [1,H] act or NULL.
 * Outputs: topk_ids [T,k] int32, descending logit (ties -> lower id);
 *          topk_w   [T,k] fp32, exp(l_j - l_max) / sum over the k chosen;
 *          shared_logit [T] fp32 = w_sg . x_t (written iff sh_gate_w and
 *          shared_logit are both non-NULL).
 * Logits are fp32: bf16 x bf16 products accumulated in fp32 (no rounding of
 * the logits to bf16).                                                      */
moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const void* sh_gate_w, int32_t* topk_ids, float* topk_w,
                     float* shared_logit, void* ws, size_t ws_bytes, void* stream);

/* Dispatch (the dispatch stage of the pipeline figure): dropless, stable
 * counting sort of the R = T*k flat assignments a = t*k + j by expert id.
 *   topk_ids [T,k] int32 in [0,E).  The router gives k distinct ids per
 *   token; repeated ids are still sorted stably (each assignment its own
 *   slot), and ids outside [0,E) are clamped into range, so the outputs are
 *   always a permutation and its inverse.
 * Outputs: expert_offsets [E+1] int32 (exclusive prefix sum of per-expert
 *          counts, offsets[E] = R); sorted_assign [R] int32 (assignments in
 *          (expert, a) order); assign_pos [R] int32 (its inverse).           */
moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_ids,
                        int32_t* expert_offsets, int32_t* sorted_assign,
                        int32_t* assign_pos, void* ws, size_t ws_bytes, void* stream);

/* Grouped expert FFN (the grouped expert GEMM stage of the figure): for
 * every dispatched row r in [offsets[e], offsets[e+1]) with token t = sorted_assign[r] / k,
 *   y[r] = expert_e(x_t)              (y [R,H] act, permuted order)
 * and, if the problem has a shared expert and y_shared != NULL,
 *   y_shared[t] = shared(x_t)         (y_shared [T,H] act).
 * Experts with few rows stream their weights once through a small-M MFMA
 * kernel; the rest run on an LDS-tiled MFMA grouped GEMM.                   */
moe_status moe_expert_ffn(const moe_problem* p, const moe_weights* w, const void* x,
                          const int32_t* expert_offsets, const int32_t* sorted_assign,
                          void* y, void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* The two grouped GEMM phases of moe_expert_ffn as separate calls (same
 * kernels; each call plans its own work lists from expert_offsets):
 *   gate/up: h[r] = SiLU(W_gate[e] x_t) * (W_up[e] x_t) for every dispatched
 *            row r (h [R, I] act, permuted order) and, if h_shared != NULL and
 *            the problem has a shared expert, h_shared[t] ([T, I_shared] act);
 *   down   : y[r] = W_down[e] h[r] (y [R, H] act) and, if y_shared and
 *            h_shared are non-NULL, y_shared[t] = S_down h_shared[t].
 * h is rounded to the activation dtype between the phases, exactly as inside
 * moe_expert_ffn.                                                            */
moe_status moe_expert_gate_up(const moe_problem* p, const moe_weights* w, const void* x,
                              const int32_t* expert_offsets, const int32_t* sorted_assign,
                              void* h, void* h_shared, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_down(const moe_problem* p, const moe_weights* w, const int32_t* expert_offsets,
                           const void* h, const void* h_shared, void* y, void* y_shared,
                           void* ws, size_t ws_bytes, void* stream);

/* Weighted combine + gated shared expert (the figure's last stage;
 * eq. MoE(x)):
 *   out[t] = sum_{j<k} topk_w[t,j] * y[assign_pos[t*k+j]]
 *            + sigmoid(shared_logit[t]) * y_shared[t]
 * in fp32, j ascending, then rounded to act dtype.  y_shared and
 * shared_logit are both NULL (no shared term) or both non-NULL.            */
moe_status moe_combine(const moe_problem* p, const void* y, const int32_t* assign_pos,
                       const float* topk_w, const void* y_shared,
                       const float* shared_logit, void* out, void* stream);

/* The whole layer: route -> dispatch -> expert FFN -> combine, with all
 * intermediates in ws.  out [T,H] act.  topk_ids / topk_w may be NULL; if
 * given they receive the routing ([T,k] int32 / fp32).                      */
moe_status moe_layer_forward(const moe_problem* p, const moe_weights* w, const void* x,
                             void* out, int32_t* topk_ids, float* topk_w,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): the same kernels, with the workspace in a device array inside
 * the library instead of the ws argument.  It calls no allocating routine.
 *   Problems whose moe_workspace_bytes(p) exceeds MOE_NOALLOC_SCRATCH_BYTES
 *   (32 MiB: decode batches and prefill chunks of a few hundred tokens at the
 *   2.4T shape) return MOE_ERR_WORKSPACE before any launch.
 *   Each GPU holds one copy of the array for the life of the process, shared
 *   by every call on that GPU: calls that overlap on one GPU (different
 *   streams or threads) race on it and must be serialised by the caller.
 *   Nothing in it needs to start at zero; every call writes what it reads.
 * Other arguments, outputs and errors as moe_layer_forward.               */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_forward_noalloc(const moe_problem* p, const moe_weights* w, const void* x,
                                     void* out, int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------------------
 * Gated residual around the layer (Qwen3.8-Flash-Next study, "Gated residual:
 * four streams, one sublayer input"): the persistent residual is four
 * streams of width H; the layer reads one gated mean of them and writes its
 * output back into each stream with a scalar gate.
 *   Rhat_i = GroupRMSNorm(R_i)           (stream i alone: R_i / sqrt(mean R_i^2 + eps) * norm_w[i])
 *   G      = sigmoid(W_up SiLU(W_down vec(Rhat) / 4))
 *   x      = mean_i (G_i * Rhat_i),   s = 2 sigmoid(W_write vec(Rhat) / 4)
 *   R'_i   = R_i + s_i F(x)              (F = the layer, e.g. moe_layer_forward)
 * bf16 activations only (MOE_ERR_UNSUPPORTED otherwise); H a multiple of 32,
 * rank a multiple of 16.  Uses p->T, p->H and p->act_dtype of the layer's
 * problem.  All pointers device memory, 16-byte aligned, caller-owned.
 * --------------------------------------------------------------------------- */
typedef struct {
  const void* norm_w; /* [4, H] bf16: RMSNorm gain of each stream                              */
  const void* w_read; /* [rank + 4, 4H] bf16: rows 0..rank-1 W_down, rows rank..rank+3 W_write */
  const void* w_up;   /* [4H, rank] bf16: the read gate's up projection                        */
  int64_t rank;       /* read bottleneck width (320 in the study)                             */
  float eps;          /* RMSNorm epsilon (rms_norm_eps 1e-6 in the model config)               */
} moe_gr_weights;

/* Scratch bytes moe_gr_read needs: Rhat [T, 4H] bf16, split-K partials of
 * the read projection, the bottleneck activations [T, rank] bf16. */
size_t moe_gr_workspace_bytes(const moe_problem* p, int64_t rank);

/* resid [T, 4, H] bf16 (stream i at columns iH .. iH+H-1 of a token) ->
 * x [T, H] bf16 (the layer's input) and s [T, 4] fp32 (write gates).
 * Errors as moe_route (shapes, alignment, workspace) before any launch. */
moe_status moe_gr_read(const moe_problem* p, const moe_gr_weights* g, const void* resid, void* x, float* s,
                       void* ws, size_t ws_bytes, void* stream);

/* resid_out [T, 4, H] = resid + s[:, i] * f (f [T, H] bf16, the layer's
 * output); resid_out may alias resid. */
moe_status moe_gr_write(const moe_problem* p, const void* resid, const float* s, const void* f, void* resid_out,
                        void* stream);

/* moe_combine and moe_gr_write in one pass: the combine's F(x) = MoE(x)
 * (rounded to bf16 as moe_combine stores it) goes straight into
 *   resid_out [T, 4, H] = resid + s[:, i] * F(x)
 * without being written and read back; the result equals moe_combine
 * followed by moe_gr_write bit for bit.  out [T, H] bf16 receives F(x) too
 * when non-NULL.  Arguments as moe_combine and moe_gr_write (y_shared and
 * shared_logit both NULL or both non-NULL); resid_out may alias resid, out
 * must not overlap resid or resid_out.  bf16 activations only
 * (MOE_ERR_UNSUPPORTED otherwise), H a multiple of 32. */
moe_status moe_combine_gr_write(const moe_problem* p, const void* y, const int32_t* assign_pos,
                                const float* topk_w, const void* y_shared, const float* shared_logit,
                                const void* resid, const float* s, void* out, void* resid_out, void* stream);

/* ---------------------------------------------------------------------------
 * Expert-weight audit (model-hub discussion "singular matrices in
 * Qwen3.8-2.4T-A95B"): for a bf16 weight tensor cut into `slices` equal
 * slices (e.g. one per expert of an [E, I, H] tensor), the number of exact
 * zeros (the discussion's "zer%" column) and the robust spread
 *   sigma_rob = 1.4826 * median(|w_i - median(w)|)
 * of each slice and of the whole tensor.  The median of an even count is the
 * mean of the two middle values; both signed zeros are zeros; a NaN in a set
 * (or an empty set) makes its median, mad and sigma_rob NaN.  The statistics
 * are exact: every value is one of the 65536 bf16 patterns, so the kernels
 * count patterns and derive the order statistics from the counts, in fp64.
 * --------------------------------------------------------------------------- */
typedef struct moe_audit_stats {
  int64_t n;        /* values in the set                                      */
  int64_t n_zero;   /* values equal to 0 (+0 or -0)                           */
  int64_t n_nan;    /* NaN values                                             */
  double median;    /* median of the values                                   */
  double mad;       /* median of |w - median|                                 */
  double sigma_rob; /* 1.4826 * mad                                           */
} moe_audit_stats;

/* Scratch bytes of moe_weight_audit: one 65536-bin uint32 histogram per
 * slice, with a table of its 1024 group counts (64 value-order positions a
 * group), and one uint64 histogram of the whole tensor.  0 if slices < 1 or
 * slices > 65535. */
size_t moe_audit_workspace_bytes(int64_t slices);

/* w: device, dtype MOE_BF16 (MOE_ERR_UNSUPPORTED otherwise); slice s is the
 * n contiguous values at w + s * slice_stride (elements; slice_stride >= n).
 * stats: device, [slices + 1] records, caller-owned: the slices in order,
 * then the whole tensor.  1 <= slices <= 65535 and n < 2^32 (MOE_ERR_SHAPE
 * otherwise); w 2-byte aligned, stats 8-byte aligned, ws 256-byte aligned
 * (MOE_ERR_ALIGN).  n == 0 is valid (every record then has n = 0 and NaN
 * statistics).  Errors are reported before any launch. */
moe_status moe_weight_audit(const void* w, int32_t dtype, int64_t slices, int64_t n, int64_t slice_stride,
                            moe_audit_stats* stats, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helper (not a step of the layer): reads `bytes` of device
 * memory at src once, 16 bytes per lane over contiguous runs with eight loads
 * in flight per lane, and writes nothing (sink: a device uint32, written only
 * in a case that does not arise in practice).  Its rate is the practical HBM
 * read ceiling that the streaming stages' rates are compared with.  src
 * 16-byte aligned and bytes a multiple of 16 (MOE_ERR_ALIGN).
 * --------------------------------------------------------------------------- */
moe_status moe_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement helper (not a step of the layer): the 256 x 256 MFMA tile
 * kernel's per-step work taken apart, one workgroup of 8 waves per CU, each
 * wave issuing 16 v_mfma_f32_32x32x16_bf16 per step on zero operands (so the
 * chip's power limit does not lower the clock) for `steps` steps; FLOPs per
 * launch = CUs x 8 x steps x 16 x 32768.  variant adds, cumulatively:
 *   0  nothing (the MFMA rate alone);
 *   1  the tile kernel's 12 16-byte LDS fragment reads per wave and step;
 *   2  one workgroup barrier per step;
 *   3  its direct loads (buffer_load ... lds, 4 x 1 KB per wave and step,
 *      32 KB per workgroup) from src, with a wait for the loads two steps old;
 *   4  variant 3 without the barrier;
 *   5  variant 3 with the loads as global_load_lds (with these in flight the
 *      compiler waits for every LDS operation before each MFMA).
 * src (variants 3-5): device, 16-byte aligned, src_bytes a nonzero multiple
 * of 32768 (at most 2^20 slots), read in 32 KB slots; ignored by variants
 * 0-2 (may be NULL).  sink: a device float, written only in a case that does
 * not arise.  MOE_ERR_SHAPE for a variant outside 0-5 or steps outside
 * [1, 2^24]; errors are reported before any launch.
 * --------------------------------------------------------------------------- */
moe_status moe_mfma_pipe_probe(int32_t variant, int32_t steps, const void* src, size_t src_bytes, float* sink,
                               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
