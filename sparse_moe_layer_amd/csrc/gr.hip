// Gated residual read and write around a sublayer (Qwen3.8-Flash-Next study,
// "Gated residual: four streams, one sublayer input"):
//   Rhat_i = GroupRMSNorm(R_i)                    per stream, gain g_i, eps
//   G      = sigmoid(W_up SiLU(W_down vec(Rhat) / 4))
//   x      = mean_i (G_i * Rhat_i),   s = 2 sigmoid(W_write vec(Rhat) / 4)
//   R'_i   = R_i + s_i F(x)
// bf16 activations and weights, fp32 arithmetic.
//
// Read: (1) gr_norm_kernel, one workgroup per token, writes Rhat [T, 4H] bf16;
// (2) the split-K MFMA router GEMM computes vec(Rhat) . [W_down; W_write]^T
// (fp32 partials over K chunks); (3) gr_gate_kernel adds the partials in
// chunk order, divides by 4 and applies SiLU (bottleneck) or 2 sigmoid (write
// gates); (4) gr_up_kernel forms W_up z on v_mfma_f32_32x32x16_bf16 and, in
// its epilogue, x = 1/4 sum_i sigmoid(.) * Rhat_i: a wave owns 32 tokens x 32
// hidden columns and computes the four streams' rows of W_up for the same
// columns (four 32x32 blocks), so G never leaves registers.
// Write: gr_write_kernel, elementwise, 16-byte vectors.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int STREAMS = 4;

__global__ __launch_bounds__(256) void gr_norm_kernel(const bf16* __restrict__ resid, const bf16* __restrict__ gain,
                                                      bf16* __restrict__ rhat, int H, float eps) {
  __shared__ float part[STREAMS][4];  // per stream, per wave
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bf16* r = resid + (int64_t)t * STREAMS * H;
  const int chunks = H / 8;  // 16-byte chunks per stream
  float ss[STREAMS] = {0.f, 0.f, 0.f, 0.f};
  for (int q = threadIdx.x; q < STREAMS * chunks; q += blockDim.x) {
    const int i = q / chunks;
    const bf16x8 v = __builtin_bit_cast(bf16x8, ld16(r + (int64_t)q * 8));
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf(bf2f(v[e]), bf2f(v[e]), a);
#pragma unroll
    for (int s = 0; s < STREAMS; ++s)
      if (s == i) ss[s] += a;
  }
#pragma unroll
  for (int s = 0; s < STREAMS; ++s) {
    const float w = wave_sum(ss[s]);
    if (lane == 0) part[s][wave] = w;
  }
  __syncthreads();
  float inv[STREAMS];
#pragma unroll
  for (int s = 0; s < STREAMS; ++s)
    inv[s] = rsqrtf((part[s][0] + part[s][1] + part[s][2] + part[s][3]) / (float)H + eps);
  bf16* o = rhat + (int64_t)t * STREAMS * H;
  for (int q = threadIdx.x; q < STREAMS * chunks; q += blockDim.x) {
    const int i = q / chunks;
    const bf16x8 v = __builtin_bit_cast(bf16x8, ld16(r + (int64_t)q * 8));
    const bf16x8 g = __builtin_bit_cast(bf16x8, ld16(gain + (int64_t)q * 8));
    float sc = inv[0];
#pragma unroll
    for (int s = 1; s < STREAMS; ++s)
      if (s == i) sc = inv[s];
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = f2bf(bf2f(v[e]) * sc * bf2f(g[e]));
    st16(o + (int64_t)q * 8, __builtin_bit_cast(u32x4, y));
  }
}

// partial [nsplit][T][rank + 4] -> z [T, rank] = SiLU(sum / 4) (bf16),
// s [T, 4] = 2 sigmoid(sum / 4); chunks added in order.
__global__ void gr_gate_kernel(const float* __restrict__ partial, int nsplit, int T, int rank,
                               bf16* __restrict__ z, float* __restrict__ s) {
  const int N = rank + STREAMS;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * N) return;
  const int t = (int)(idx / N), n = (int)(idx % N);
  float a = 0.f;
  for (int c = 0; c < nsplit; ++c) a += partial[((int64_t)c * T + t) * N + n];
  a *= 0.25f;
  if (n < rank) z[(int64_t)t * rank + n] = f2bf(silu(a));
  else s[(int64_t)t * STREAMS + (n - rank)] = 2.0f * sigmoid(a);
}

// x[t, c] = 1/4 sum_i sigmoid(z[t] . W_up[i*H + c]) * Rhat[t, i*H + c].
// Workgroup: 4 waves = 128 tokens x 32 columns; wave w: tokens t0 + 32w ..,
// four 32x32 blocks (one per stream).  Operand fragments come straight from
// global memory (z and W_up stay in L2): A lane = token lane%32, K values
// 8*(lane/32) ..; B lane = W_up row lane%32 of the block, same K values.
__global__ __launch_bounds__(256) void gr_up_kernel(const bf16* __restrict__ z, const bf16* __restrict__ w_up,
                                                    const bf16* __restrict__ rhat, bf16* __restrict__ x, int T, int H,
                                                    int rank) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 128 + wave * 32;
  const int c0 = blockIdx.y * 32;
  int ta = t0 + (lane & 31);
  ta = ta < T ? ta : T - 1;  // rows past T: computed, never stored
  const bf16* arow = z + (int64_t)ta * rank + 8 * (lane >> 5);
  const bf16* brow[STREAMS];
#pragma unroll
  for (int i = 0; i < STREAMS; ++i) brow[i] = w_up + (int64_t)(i * H + c0 + (lane & 31)) * rank + 8 * (lane >> 5);
  f32x16 acc[STREAMS];
#pragma unroll
  for (int i = 0; i < STREAMS; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  for (int k = 0; k < rank; k += 16) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(arow + k));
#pragma unroll
    for (int i = 0; i < STREAMS; ++i) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(brow[i] + k));
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
    }
  }
  // C lane layout: column lane%32, rows 8*(v/4) + 4*(lane/32) + v%4
  const int c = c0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (t >= T) continue;
    const bf16* rh = rhat + (int64_t)t * STREAMS * H + c;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < STREAMS; ++i) sum += sigmoid(acc[i][v]) * bf2f(rh[(int64_t)i * H]);
    x[(int64_t)t * H + c] = f2bf(0.25f * sum);
  }
}

// out may alias resid: each element is read and then written by one thread.
__global__ void gr_write_kernel(const bf16* resid, const float* __restrict__ s, const bf16* __restrict__ f,
                                bf16* out, int T, int H) {
  const int chunks = H / 8;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, i, chunk)
  if (q >= (int64_t)T * STREAMS * chunks) return;
  const int64_t t = q / (STREAMS * chunks);
  const int i = (int)((q / chunks) % STREAMS);
  const int c = (int)(q % chunks);
  const float si = s[t * STREAMS + i];
  const bf16x8 r = __builtin_bit_cast(bf16x8, ld16(resid + q * 8));
  const bf16x8 fv = __builtin_bit_cast(bf16x8, ld16(f + t * H + (int64_t)c * 8));
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f2bf(fmaf(si, bf2f(fv[e]), bf2f(r[e])));
  st16(out + q * 8, __builtin_bit_cast(u32x4, o));
}

}  // namespace

size_t gr_workspace_bytes(int64_t T, int64_t H, int64_t rank) {
  const int nsplit = router_gemm_split((int)T, (int)(STREAMS * H), (int)(rank + STREAMS));
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up((size_t)T * STREAMS * H * 2) + up((size_t)nsplit * T * (rank + STREAMS) * 4) + up((size_t)T * rank * 2);
}

hipError_t launch_gr_read(const void* resid, const void* norm_w, const void* w_read, const void* w_up, float eps,
                          int T, int H, int rank, void* x, float* s, void* ws, hipStream_t st) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  char* w = static_cast<char*>(ws);
  bf16* rhat = reinterpret_cast<bf16*>(w);
  w += up((size_t)T * STREAMS * H * 2);
  const int N = rank + STREAMS;
  const int nsplit = router_gemm_split(T, STREAMS * H, N);
  float* partial = reinterpret_cast<float*>(w);
  w += up((size_t)nsplit * T * N * 4);
  bf16* z = reinterpret_cast<bf16*>(w);
  gr_norm_kernel<<<T, 256, 0, st>>>(reinterpret_cast<const bf16*>(resid), reinterpret_cast<const bf16*>(norm_w), rhat,
                                    H, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_router_logits_bf16(rhat, w_read, nullptr, partial, T, STREAMS * H, N, nsplit, st);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)T * N;
  gr_gate_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(partial, nsplit, T, rank, z, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  gr_up_kernel<<<dim3((T + 127) / 128, H / 32), 256, 0, st>>>(z, reinterpret_cast<const bf16*>(w_up), rhat,
                                                              reinterpret_cast<bf16*>(x), T, H, rank);
  return hipGetLastError();
}

hipError_t launch_gr_write(const void* resid, const float* s, const void* f, void* out, int T, int H,
                           hipStream_t st) {
  const int64_t n = (int64_t)T * STREAMS * (H / 8);
  gr_write_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<const bf16*>(resid), s,
                                                               reinterpret_cast<const bf16*>(f),
                                                               reinterpret_cast<bf16*>(out), T, H);
  return hipGetLastError();
}

}  // namespace moe
