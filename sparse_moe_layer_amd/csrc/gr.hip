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
// gates); (4) the up projection (gr_up_lds_kernel, LDS-tiled, from 64 tokens;
// gr_up_kernel below that) forms W_up z on v_mfma_f32_32x32x16_bf16 and, in
// its epilogue, x = 1/4 sum_i sigmoid(.) * Rhat_i: a wave owns 32 tokens x 32
// hidden columns and computes the four streams' rows of W_up for the same
// columns (four 32x32 blocks), so G never leaves registers.
// Write: gr_write_kernel, elementwise, 16-byte vectors.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int STREAMS = 4;
constexpr int kUpBatchedMinT = 64;  // token count from which the LDS-tiled up projection is used
constexpr int kUpBK = 64;           // K values per LDS slice of the up projection

// One workgroup per token: the sum of squares of each stream, then the
// scaled row (the second pass re-reads the token's row, which is still in L2;
// holding it in registers instead measured slower, by occupancy).
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

template <int BATCH>
__device__ __forceinline__ float sum_chunks(const float* col, int64_t cs, int nsplit) {
  float a = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += BATCH) {
    float p[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) p[j] = c0 + j < nsplit ? col[(c0 + j) * cs] : 0.f;
#pragma unroll
    for (int j = 0; j < BATCH; ++j) a += p[j];
  }
  return a;
}

// partial [nsplit][T][rank + 4] -> z [T, rank] = SiLU(sum / 4) (bf16),
// s [T, 4] = 2 sigmoid(sum / 4).
__global__ void gr_gate_kernel(const float* __restrict__ partial, int nsplit, int T, int rank,
                               bf16* __restrict__ z, float* __restrict__ s) {
  const int N = rank + STREAMS;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * N) return;
  const int t = (int)(idx / N), n = (int)(idx % N);
  // all chunk loads of a batch in flight at once, added in chunk order
  const float* col = partial + (int64_t)t * N + n;
  const int64_t cs = (int64_t)T * N;
  const float a = 0.25f * (nsplit <= 8 ? sum_chunks<8>(col, cs, nsplit) : sum_chunks<32>(col, cs, nsplit));
  if (n < rank) z[(int64_t)t * rank + n] = f2bf(silu(a));
  else s[(int64_t)t * STREAMS + (n - rank)] = 2.0f * sigmoid(a);
}

// Epilogue of the up projection for one wave's 32 tokens (from tw) x one
// column c per lane: acc[i] holds the stream-i gate logits in the 32x32 MFMA
// C layout (column lane % 32, rows 8 (v / 4) + 4 (lane / 32) + v % 4).  All 64
// Rhat values are loaded before any is used (rows past T read row T - 1 and
// are not stored), so their latency is paid once.
__device__ __forceinline__ void gated_mean_store(const f32x16 (&acc)[STREAMS], const bf16* __restrict__ rhat,
                                                 bf16* __restrict__ x, int tw, int c, int lane, int T, int H) {
  bf16 rv[16][STREAMS];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    int t = tw + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    t = t < T ? t : T - 1;
    const bf16* rh = rhat + (int64_t)t * STREAMS * H + c;
#pragma unroll
    for (int i = 0; i < STREAMS; ++i) rv[v][i] = rh[(int64_t)i * H];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = tw + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < STREAMS; ++i) sum += sigmoid(acc[i][v]) * bf2f(rv[v][i]);
    if (t < T) x[(int64_t)t * H + c] = f2bf(0.25f * sum);
  }
}

// x[t, c] = 1/4 sum_i sigmoid(z[t] . W_up[i*H + c]) * Rhat[t, i*H + c].
//
// Batched form: a workgroup owns 128 tokens x 32 hidden columns; its operand
// tiles (128 rows of z, and the 4 x 32 rows of W_up that give the four
// streams' gates for those columns) pass through LDS BK K values at a time,
// double buffered (the next slice is loaded into registers while the MFMAs
// run on the current one).  Wave w computes tokens 32w .. 32w+31 against all four
// streams, so the gated mean is formed in registers.  Workgroup b runs on
// XCD b % 8; when the column blocks split evenly, each XCD takes one eighth of
// the columns (its W_up slice stays in that XCD's L2) and walks the token
// blocks, all of its column blocks of one token block in turn.
constexpr int UP_BT = 128;

template <int BK>
struct UpTile {
  static constexpr int CPR = BK / 8;             // 16-byte chunks per LDS row
  static constexpr int LOADS = UP_BT * CPR / 256;  // chunks per thread per tile per slice
  static constexpr int RSTEP = 256 / CPR;          // rows between a thread's chunks
  // chunk c of row r sits at c ^ f(r), so that the 16 lanes of a 128-bit
  // LDS access (16 consecutive rows, one chunk) touch 64 distinct banks
  __device__ static int pos(int r, int c) {
    return r * CPR + (CPR == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3)));
  }
};

template <int BK>
__global__ __launch_bounds__(256, BK == 64 ? 2 : 3) void gr_up_lds_kernel(const bf16* __restrict__ z,
                                                                          const bf16* __restrict__ w_up,
                                                                          const bf16* __restrict__ rhat,
                                                                          bf16* __restrict__ x, int T, int H,
                                                                          int rank) {
  using U = UpTile<BK>;
  __shared__ u32x4 sa[2][UP_BT * U::CPR];
  __shared__ u32x4 sb[2][STREAMS * 32 * U::CPR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n_cb = H / 32;
  const int b = blockIdx.x;
  int tb, cb;
  if ((n_cb & 7) == 0) {
    const int cpx = n_cb >> 3, slot = b >> 3;
    cb = (b & 7) * cpx + slot % cpx;
    tb = slot / cpx;
  } else {
    tb = b / n_cb;
    cb = b % n_cb;
  }
  const int t0 = tb * UP_BT, c0 = cb * 32;
  // this thread's chunks of each tile per slice: rows tid / CPR + RSTEP j, chunk tid % CPR
  const int ch = tid % U::CPR;
  const bf16* ga[U::LOADS];
  const bf16* gb[U::LOADS];
  int so[U::LOADS];
#pragma unroll
  for (int j = 0; j < U::LOADS; ++j) {
    const int row = tid / U::CPR + U::RSTEP * j;
    int t = t0 + row;
    t = t < T ? t : T - 1;  // rows past T: computed, never stored
    ga[j] = z + (int64_t)t * rank + ch * 8;
    gb[j] = w_up + (int64_t)((row >> 5) * H + c0 + (row & 31)) * rank + ch * 8;
    so[j] = U::pos(row, ch);
  }
  u32x4 ra[U::LOADS], rb[U::LOADS];
  auto load = [&](int k0) {
    const bool in = k0 + ch * 8 < rank;  // rank % 16 == 0: a chunk is all in or all out
#pragma unroll
    for (int j = 0; j < U::LOADS; ++j) {
      ra[j] = in ? ld16(ga[j] + k0) : u32x4{0u, 0u, 0u, 0u};
      rb[j] = in ? ld16(gb[j] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < U::LOADS; ++j) {
      sa[buf][so[j]] = ra[j];
      sb[buf][so[j]] = rb[j];
    }
  };
  f32x16 acc[STREAMS];
#pragma unroll
  for (int i = 0; i < STREAMS; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
  const int nk = (rank + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  const int ar = wave * 32 + (lane & 31);
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) load((it + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);  // K values 16 kk + 8 (lane / 32) ..
      const bf16x8 a = __builtin_bit_cast(bf16x8, sa[cur][U::pos(ar, c)]);
#pragma unroll
      for (int i = 0; i < STREAMS; ++i) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, sb[cur][U::pos(i * 32 + (lane & 31), c)]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[i], 0, 0, 0);
      }
    }
    // buffer cur ^ 1 was last read before the previous barrier
    if (it + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  gated_mean_store(acc, rhat, x, t0 + wave * 32, c0 + (lane & 31), lane, T, H);
}

// Few tokens: the same product with operand fragments read straight from
// global memory (z and W_up stay in L2), one workgroup per 128 tokens x 32
// columns as above but without the LDS tiles, so that a handful of tokens
// does not pay for 128-row tile loads.
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
  gated_mean_store(acc, rhat, x, t0, c0 + (lane & 31), lane, T, H);
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

// The read projection's K split may run in more rounds than the router's:
// its K is 4H, and 8 chunks (two rounds plus) cut the 2.4T-shape read from
// 0.97 to 0.94 ms; its partial sums are read once by the gate kernel.
constexpr int kGrMaxSplit = 8;

size_t gr_workspace_bytes(int64_t T, int64_t H, int64_t rank) {
  const int nsplit = router_gemm_split((int)T, (int)(STREAMS * H), (int)(rank + STREAMS), kGrMaxSplit);
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
  const int nsplit = router_gemm_split(T, STREAMS * H, N, kGrMaxSplit);
  float* partial = reinterpret_cast<float*>(w);
  w += up((size_t)nsplit * T * N * 4);
  bf16* z = reinterpret_cast<bf16*>(w);
  gr_norm_kernel<<<T, 256, 0, st>>>(reinterpret_cast<const bf16*>(resid), reinterpret_cast<const bf16*>(norm_w), rhat,
                                    H, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_router_logits_bf16(rhat, w_read, nullptr, partial, T, STREAMS * H, N, nsplit, st, true);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)T * N;
  gr_gate_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(partial, nsplit, T, rank, z, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (T >= kUpBatchedMinT)
    gr_up_lds_kernel<kUpBK><<<((T + UP_BT - 1) / UP_BT) * (H / 32), 256, 0, st>>>(
        z, reinterpret_cast<const bf16*>(w_up), rhat, reinterpret_cast<bf16*>(x), T, H, rank);
  else
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
