// Weighted combine + gated shared expert (Qwen3.8-Flash-Next study, MoE
// section: the last stage of the pipeline figure and eq. MoE(x)):
//   out[t] = sum_{j<k} w[t,j] * y[pos[t*k+j]] + sigmoid(s_t) * y_shared[t]
// 16-byte loads of y rows (8 bf16 or 4 fp32 per thread), fp32 accumulation
// with j ascending, one rounding to the output dtype.  HBM-bound: reads k+1
// rows of H and writes one.  Every row is read once, so the loads are
// non-temporal (2.4T-shape prefill combine 0.321 -> 0.273 ms).
//
// With the gated residual around the layer (same study, "Gated residual:
// four streams, one sublayer input"), the stream write R'_i = R_i + s_i F(x)
// can run in the combine's epilogue: the thread that rounds F(x) for 8
// columns of token t updates the same 8 columns of the token's four
// streams, so F(x) need not be written and read back.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// acc[0..VEC) += wgt * (16 bytes of y: 4 fp32 or 8 bf16)
template <bool F32>
__device__ __forceinline__ void accumulate(float* acc, float wgt, u32x4 v) {
  if constexpr (F32) {
    const f32x4 f = __builtin_bit_cast(f32x4, v);  // whole-vector cast (not per element)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wgt, f[i], acc[i]);
  } else {
    const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wgt, bf2f(b[i]), acc[i]);
  }
}

// Workgroup (t, blockIdx.y) covers 16-byte chunks blockIdx.y*256 + tid of
// token t.  The token's k row positions and weights are the same for the
// whole workgroup (scalar loads); a thread issues the y rows of the token's
// assignments and the shared expert's row at once, then adds them (j
// ascending, the shared expert last), so the k+1 row reads overlap instead
// of forming a chain.  KB > 0: k <= KB, one batch, every load unconditional
// (indices clamped into the token's k); KB == 0: any k, batches of 16.
// GRW (bf16 only): the gated-residual stream write in the epilogue;
// resid / s / resid_out as gr_write (resid_out may alias resid: each element
// is read and then written by one thread), out may be null.
template <bool F32, bool GRW, int KB>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, const void* __restrict__ y_sh,
                                                      const float* __restrict__ sl, void* __restrict__ out, int H,
                                                      int k, const bf16* resid, const float* __restrict__ s,
                                                      bf16* resid_out) {
  static_assert(!(F32 && GRW), "the gated residual is bf16");
  constexpr int VEC = F32 ? 4 : 8;
  constexpr int ESZ = F32 ? 4 : 2;
  const int t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= H / VEC) return;
  const int64_t col = (int64_t)c * VEC;
  const char* yb = reinterpret_cast<const char*>(y);
  const int32_t* pt = pos + (int64_t)t * k;
  const float* wt = w + (int64_t)t * k;
  constexpr int STREAMS = 4;
  u32x4 r[GRW ? STREAMS : 1];
  if constexpr (GRW) {
#pragma unroll
    for (int i = 0; i < STREAMS; ++i) r[i] = ld16_nt(resid + ((int64_t)t * STREAMS + i) * H + col);
  }
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  if constexpr (KB > 0) {
    // without a shared expert its load reads row 0 of y instead (unused)
    const char* shp = y_sh ? reinterpret_cast<const char*>(y_sh) + (int64_t)t * H * ESZ : yb;
    const u32x4 vsh = ld16_nt(shp + col * ESZ);
    int64_t row[KB];
    float wj[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int j = b < k ? b : k - 1;
      row[b] = (int64_t)pt[j] * H;
      wj[b] = wt[j];
    }
    u32x4 v[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) v[b] = ld16_nt(yb + (row[b] + col) * ESZ);
#pragma unroll
    for (int b = 0; b < KB; ++b)
      if (b < k) accumulate<F32>(acc, wj[b], v[b]);
    if (y_sh) accumulate<F32>(acc, sigmoid(sl[t]), vsh);
  } else {
    u32x4 vsh = {0, 0, 0, 0};
    if (y_sh) vsh = ld16_nt(reinterpret_cast<const char*>(y_sh) + ((int64_t)t * H + col) * ESZ);
    for (int j0 = 0; j0 < k; j0 += 16) {
      u32x4 v[16];
#pragma unroll
      for (int b = 0; b < 16; ++b)
        if (j0 + b < k) v[b] = ld16_nt(yb + ((int64_t)pt[j0 + b] * H + col) * ESZ);
#pragma unroll
      for (int b = 0; b < 16; ++b)
        if (j0 + b < k) accumulate<F32>(acc, wt[j0 + b], v[b]);
    }
    if (y_sh) accumulate<F32>(acc, sigmoid(sl[t]), vsh);
  }
  char* dst = out ? reinterpret_cast<char*>(out) + ((int64_t)t * H + col) * ESZ : nullptr;
  if constexpr (F32) {
    st16(dst, __builtin_bit_cast(u32x4, f32x4{acc[0], acc[1], acc[2], acc[3]}));
  } else {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f2bf(acc[i]);
    if (dst) st16(dst, __builtin_bit_cast(u32x4, o));
    if constexpr (GRW) {
      // R'_i = R_i + s_i F(x) with F(x) rounded as stored, as gr_write does
#pragma unroll
      for (int i = 0; i < STREAMS; ++i) {
        const float si = s[(int64_t)t * STREAMS + i];
        const bf16x8 rv = __builtin_bit_cast(bf16x8, r[i]);
        bf16x8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = f2bf(fmaf(si, bf2f(o[e]), bf2f(rv[e])));
        st16(resid_out + ((int64_t)t * STREAMS + i) * H + col, __builtin_bit_cast(u32x4, ov));
      }
    }
  }
}

}  // namespace

// One batch of KB row loads: the smallest of 1, 2, 4, 8, 10, 12, 16 that
// covers k (the common k load no row twice); k > 16: batches of 16.
#define MOE_COMBINE_KB(F32, GRW, ...)                                                             \
  do {                                                                                           \
    if (k <= 1) combine_kernel<F32, GRW, 1><<<grid, 256, 0, s>>>(__VA_ARGS__);                   \
    else if (k <= 2) combine_kernel<F32, GRW, 2><<<grid, 256, 0, s>>>(__VA_ARGS__);              \
    else if (k <= 4) combine_kernel<F32, GRW, 4><<<grid, 256, 0, s>>>(__VA_ARGS__);              \
    else if (k <= 8) combine_kernel<F32, GRW, 8><<<grid, 256, 0, s>>>(__VA_ARGS__);              \
    else if (k <= 10) combine_kernel<F32, GRW, 10><<<grid, 256, 0, s>>>(__VA_ARGS__);            \
    else if (k <= 12) combine_kernel<F32, GRW, 12><<<grid, 256, 0, s>>>(__VA_ARGS__);            \
    else if (k <= 16) combine_kernel<F32, GRW, 16><<<grid, 256, 0, s>>>(__VA_ARGS__);            \
    else combine_kernel<F32, GRW, 0><<<grid, 256, 0, s>>>(__VA_ARGS__);                          \
  } while (0)

hipError_t launch_combine(const void* y, const int32_t* pos, const float* w, const void* y_sh,
                          const float* shared_logit, void* out, int T, int H, int k, int f32, hipStream_t s) {
  const int vec = f32 ? 4 : 8;
  const dim3 grid(T, (H / vec + 255) / 256);
  if (f32) MOE_COMBINE_KB(true, false, y, pos, w, y_sh, shared_logit, out, H, k, nullptr, nullptr, nullptr);
  else MOE_COMBINE_KB(false, false, y, pos, w, y_sh, shared_logit, out, H, k, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_combine_gr_write(const void* y, const int32_t* pos, const float* w, const void* y_sh,
                                   const float* shared_logit, void* out, const void* resid, const float* gate,
                                   void* resid_out, int T, int H, int k, hipStream_t s) {
  const dim3 grid(T, (H / 8 + 255) / 256);
  MOE_COMBINE_KB(false, true, y, pos, w, y_sh, shared_logit, out, H, k, reinterpret_cast<const bf16*>(resid), gate,
                 reinterpret_cast<bf16*>(resid_out));
  return hipGetLastError();
}
#undef MOE_COMBINE_KB

}  // namespace moe
