// Expert-weight audit (model-hub discussion "singular matrices in
// Qwen3.8-2.4T-A95B"): per slice of a bf16 weight tensor (e.g. per expert)
// and over the whole tensor, the number of exact zeros (the table's "zer%")
// and sigma_rob = 1.4826 * median(|w - median(w)|) (the discussion's robust
// spread), with the median of an even count the mean of the two middle values.
//
// A bf16 value is one of 65536 bit patterns, so one streaming pass that
// counts every pattern gives the exact multiset of each slice:
//   audit_hist_kernel     streams the tensor once (16-byte loads) and counts
//                         patterns: zeros in registers, 2^-63 <= |w| < 2
//                         (exponent field 64..127: 16384 patterns with the
//                         sign) in a 64 KB LDS histogram, the rare rest with
//                         global atomics; each workgroup then adds its
//                         non-empty LDS bins into the slice's histogram and
//                         the whole tensor's (uint64) in HBM, and the count
//                         of each 64-position group in value order into the
//                         slice's group table (a wave's 64 LDS bins are one
//                         group).
//                         Two workgroups share a CU, so one's flush overlaps
//                         the other's stream.
//   audit_finalize_kernel one workgroup per histogram (the slices' and the
//                         tensor's in one launch).  A slice's workgroup takes
//                         the group counts from the group table and reads
//                         only occupied groups of the histogram; the
//                         tensor's reads its whole histogram once for them
//                         (a tensor-wide table would put every workgroup's
//                         flush on the same few addresses).  Positions o in value
//                         order (-inf .. -0 | +0 .. +inf, NaN patterns at
//                         both ends) are dealt 8192 per wave; wave scans and
//                         a scan of the wave sums turn each histogram, in place,
//                         into inclusive counts in value order (stored at
//                         each position's own pattern), and the lanes
//                         holding ranks (n-1)/2 and n/2 give the median m in
//                         fp64.  Distances |v - m| are non-decreasing in o
//                         above m and non-increasing below it, so the number
//                         of values within distance D of m is two binary
//                         searches over o plus two reads of the counts; the
//                         k-th smallest distance is the least occupied
//                         position's distance D with at least k+1 values
//                         within D (a workgroup minimum), and the MAD is the
//                         mean of the two middle ones.
// Every distance is the same fp64 |v - m| that a direct evaluation forms,
// so the statistics are exact.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBins = 65536;       // bf16 bit patterns
constexpr int kLdsBins = 16384;    // patterns with exponent field 64..127, sign included
constexpr int kHistThreads = 1024;
constexpr int kFinThreads = 512;   // four finalize workgroups fit on a CU
constexpr int kOrdFirst = 0x7F;    // value-order position of -inf (below it: negative NaNs)
constexpr int kOrdLast = 0xFF80;   // +inf (above it: positive NaNs)
constexpr int kOrdZero = 0x8000;   // +0, which holds the count of every zero
constexpr int kGroups = kBins / 64; // 64-position groups in value order
constexpr double kSigmaRobScale = 1.4826;

// value order <-> pattern: negative patterns in descending magnitude, then
// the positive ones in ascending order
__device__ __forceinline__ int pat_of_ord(int o) { return o < 0x8000 ? (0x8000 | (0x7FFF - o)) : (o - 0x8000); }
__device__ __forceinline__ int ord_of_pat(uint32_t v) { return (v & 0x8000u) ? 0x7FFF - (int)(v & 0x7FFFu) : (int)v + 0x8000; }
__device__ __forceinline__ double val_of_ord(int o) {
  return (double)__uint_as_float((uint32_t)pat_of_ord(o) << 16);
}

// Inclusive scan over the 64 lanes of a wave.
template <typename CT>
__device__ __forceinline__ CT wave_incl_scan(CT v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const CT t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

template <typename CT>
__device__ __forceinline__ CT wave_total(CT v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ void audit_clear_kernel(uint32_t* __restrict__ hist, int64_t n32, unsigned long long* __restrict__ whole,
                                   uint32_t* __restrict__ grp, int64_t g32) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < n32; j += step) hist[j] = 0u;
  for (int64_t j = i; j < kBins; j += step) whole[j] = 0ull;
  for (int64_t j = i; j < g32; j += step) grp[j] = 0u;
}

__global__ __launch_bounds__(kHistThreads) void audit_hist_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                                  int64_t stride, uint32_t* __restrict__ hist,
                                                                  unsigned long long* __restrict__ whole,
                                                                  uint32_t* __restrict__ grp) {
  __shared__ uint32_t lds[kLdsBins];
  __shared__ uint32_t zsum;
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsBins; i += kHistThreads) lds[i] = 0u;
  if (tid == 0) zsum = 0u;
  __syncthreads();
  const int slice = blockIdx.y, B = gridDim.x, b = blockIdx.x;
  uint32_t* gh = hist + (int64_t)slice * kBins;
  uint32_t* gg = grp + (int64_t)slice * kGroups;
  const int lane = tid & 63;
  const uint16_t* p = w + (int64_t)slice * stride;
  // this workgroup's element range, cut at multiples of 8 elements
  const int64_t units = (n + 7) / 8;
  const int64_t lo = units * b / B * 8;
  int64_t hi = units * (b + 1) / B * 8;
  hi = hi < n ? hi : n;
  uint32_t zeros = 0;
  auto one = [&](uint32_t v) {
    if ((v & 0x7FFFu) == 0u) {
      ++zeros;
    } else if ((v & 0x6000u) == 0x2000u) {  // exponent field 64..127: 2^-63 <= |w| < 2
      atomicAdd(&lds[((v >> 15) << 13) | (v & 0x1FFFu)], 1u);
    } else {
      __hip_atomic_fetch_add(gh + v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(whole + v, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(gg + (ord_of_pat(v) >> 6), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (lo < hi) {
    // scalar head up to 16-byte alignment, 16-byte body, scalar tail
    const int64_t mis = (int64_t)((16u - (uint32_t)(reinterpret_cast<uintptr_t>(p + lo) & 15u)) & 15u) / 2;
    const int64_t body = lo + mis < hi ? lo + mis : hi;
    for (int64_t j = lo + tid; j < body; j += kHistThreads) one(p[j]);
    const int64_t nch = (hi - body) / 8;
    const u32x4* q = reinterpret_cast<const u32x4*>(p + body);
    constexpr int U = 8;  // chunks in flight per thread (8 measured 6% faster than 4)
    for (int64_t c = tid; c < nch; c += (int64_t)U * kHistThreads) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t cu = c + (int64_t)u * kHistThreads;
        v[u] = cu < nch ? __builtin_nontemporal_load(q + cu) : u32x4{0x3F80u, 0x3F80u, 0x3F80u, 0x3F80u};  // placeholder, skipped below
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c + (int64_t)u * kHistThreads >= nch) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          one(v[u][e] & 0xFFFFu);
          one(v[u][e] >> 16);
        }
      }
    }
    for (int64_t j = body + nch * 8 + tid; j < hi; j += kHistThreads) one(p[j]);
  }
  if (zeros) atomicAdd(&zsum, zeros);
  __syncthreads();
  // a wave's 64 consecutive LDS bins are 64 consecutive patterns from a
  // multiple of 64, which is one 64-position group in value order
  static_assert(kHistThreads % 64 == 0 && kLdsBins % kHistThreads == 0, "whole waves over the LDS bins");
  for (int i = tid; i < kLdsBins; i += kHistThreads) {
    const uint32_t c = lds[i];
    const int pat = ((i >> 13) << 15) | 0x2000 | (i & 0x1FFF);
    if (c) {
      __hip_atomic_fetch_add(gh + pat, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(whole + pat, (unsigned long long)c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (__ballot(c != 0)) {
      const uint32_t gs = wave_total<uint32_t>(c);
      if (lane == 0)
        __hip_atomic_fetch_add(gg + (ord_of_pat((uint32_t)pat) >> 6), gs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (tid == 0 && zsum) {
    __hip_atomic_fetch_add(gh, zsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(whole, (unsigned long long)zsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(gg + (kOrdZero >> 6), zsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ unsigned long long dbits(double d) { return (unsigned long long)__double_as_longlong(d); }

// Statistics of one histogram h (in place: the occupied groups become
// value-order prefix counts) with its group table gtab (values in each
// 64-position group), or, with gtab null, the group counts taken from h.
// A group with no values is not read again, and its prefix count lives in
// LDS.
template <typename CT>
__device__ void finalize_one(CT* __restrict__ h, const CT* __restrict__ gtab, moe_audit_stats* __restrict__ out) {
  constexpr int kWaves = kFinThreads / 64;
  constexpr int kGpw = kGroups / kWaves;        // groups per wave
  constexpr int kGpt = kGroups / kFinThreads;   // groups per thread in the group scan
  __shared__ CT gsum[kGroups];  // values in each group
  __shared__ CT gpre[kGroups];  // values in the groups before it
  __shared__ CT wsum[kWaves];
  __shared__ unsigned long long nan_sum;
  __shared__ int ord_k[2];
  __shared__ unsigned long long dmin[2];
  __shared__ unsigned long long zero_cnt;
  __shared__ int srch[3][4];  // MAD search: first passing chunk, per round and search
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    nan_sum = 0ull;
    ord_k[0] = ord_k[1] = -1;
    dmin[0] = dmin[1] = ~0ull;
    zero_cnt = 0ull;
  }
  __syncthreads();
  // pass 1: every group's count.  NaN patterns take no place in the order:
  // they sit below kOrdFirst (groups 0 and 1) and above kOrdLast (groups
  // 1022 and 1023), and are counted apart.
  if (gtab) {
    for (int g = tid; g < kGroups; g += kFinThreads) gsum[g] = gtab[g];
    __syncthreads();
    if (wave == 0) {  // the four edge groups
      unsigned long long nans = 0;
      for (int e = 0; e < 4; ++e) {
        const int g = e < 2 ? e : kGroups - 4 + e;
        if (gsum[g] == 0) continue;  // wave-uniform
        const int o = 64 * g + lane;
        const CT c = (o < kOrdFirst || o > kOrdLast) ? h[pat_of_ord(o)] : (CT)0;
        const CT tot = wave_total<CT>(c);
        nans += (unsigned long long)tot;
        if (lane == 0) gsum[g] -= tot;
      }
      if (lane == 0) nan_sum = nans;
    }
  } else {
    // wave w reads groups kGpw w ..; in its j-th step lane l takes position
    // 64 (kGpw w + j) + l, so every access is one coalesced run
    const int g0 = wave * kGpw;
    unsigned long long nans = 0;
    for (int j0 = 0; j0 < kGpw; j0 += 16) {
      CT cb[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) cb[j] = h[pat_of_ord(64 * (g0 + j0 + j) + lane)];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int o = 64 * (g0 + j0 + j) + lane;
        CT c = cb[j];
        if (o < kOrdFirst || o > kOrdLast) {
          nans += (unsigned long long)c;
          c = 0;
        }
        const CT gs = __ballot(c != 0) ? wave_total<CT>(c) : (CT)0;
        if (lane == 0) gsum[g0 + j0 + j] = gs;
      }
    }
    if (nans) atomicAdd(&nan_sum, nans);
  }
  __syncthreads();
  // exclusive prefix of the group counts: thread t holds groups kGpt t ..
  {
    CT v[kGpt], sum = 0;
#pragma unroll
    for (int i = 0; i < kGpt; ++i) {
      v[i] = gsum[kGpt * tid + i];
      sum += v[i];
    }
    const CT incl = wave_incl_scan<CT>(sum, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    CT run = incl - sum;
    for (int i = 0; i < wave; ++i) run += wsum[i];
#pragma unroll
    for (int i = 0; i < kGpt; ++i) {
      gpre[kGpt * tid + i] = run;
      run += v[i];
    }
  }
  __syncthreads();
  CT total = 0;
  for (int i = 0; i < kWaves; ++i) total += wsum[i];
  const unsigned long long n = (unsigned long long)total;
  const unsigned long long k1 = n ? (n - 1) / 2 : 0, k2 = n / 2;
  // pass 2, occupied groups only, eight groups' loads in flight together:
  // counts -> inclusive counts in value order, in place (stored at each
  // position's own pattern); find the positions of ranks k1 and k2.  The
  // occupied groups cluster around the median, so here wave w takes groups
  // w, w + kWaves, ... to share them out.
  for (int j0 = 0; j0 < kGpw; j0 += 8) {
    CT cb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = (j0 + j) * kWaves + wave;
      const int o = 64 * g + lane;
      cb[j] = (gsum[g] == 0 || o < kOrdFirst || o > kOrdLast) ? (CT)0 : h[pat_of_ord(o)];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int g = (j0 + j) * kWaves + wave;
      if (gsum[g] == 0) continue;  // wave-uniform
      const int o = 64 * g + lane;
      const CT c = cb[j];
      const CT at = gpre[g] + wave_incl_scan<CT>(c, lane);  // values at positions <= o
      if (o == kOrdZero) zero_cnt = (unsigned long long)c;
      if (c) {
        if ((unsigned long long)(at - c) <= k1 && k1 < (unsigned long long)at) ord_k[0] = o;
        if ((unsigned long long)(at - c) <= k2 && k2 < (unsigned long long)at) ord_k[1] = o;
      }
      h[pat_of_ord(o)] = at;
    }
  }
  __syncthreads();
  const unsigned long long n_nan = nan_sum;
  const double qnan = __longlong_as_double(0x7ff8000000000000ll);
  double med = qnan, mad = qnan;
  if (n > 0 && n_nan == 0) {
    med = (val_of_ord(ord_k[0]) + val_of_ord(ord_k[1])) * 0.5;
    if (__builtin_isfinite(med)) {  // an infinite or NaN median (inf - inf) leaves the MAD NaN
      const double m = med;
      // P(o): values at positions <= o (0 below the first position); an
      // empty group's positions all hold its prefix
      auto P = [&](int o) -> unsigned long long {
        if (o < kOrdFirst) return 0ull;
        o = o > kOrdLast ? kOrdLast : o;
        const int g = o >> 6;
        return gsum[g] == 0 ? (unsigned long long)gpre[g] : (unsigned long long)h[pat_of_ord(o)];
      };
      // om: first position with value >= m (values increase with o)
      int lo = kOrdFirst, hi = kOrdLast + 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (val_of_ord(mid) >= m) hi = mid;
        else lo = mid + 1;
      }
      const int om = lo;
      const unsigned long long below_all = P(om - 1);
      // values within distance D of m
      auto within = [&](double D) -> unsigned long long {
        // above: last o >= om with v - m <= D
        int a = om, b = kOrdLast + 1;
        while (a < b) {
          const int mid = (a + b) >> 1;
          if (__builtin_fabs(val_of_ord(mid) - m) <= D) a = mid + 1;
          else b = mid;
        }
        const unsigned long long above = P(a - 1) - below_all;
        // below: first o < om with m - v <= D
        int c = kOrdFirst, d = om;
        while (c < d) {
          const int mid = (c + d) >> 1;
          if (__builtin_fabs(val_of_ord(mid) - m) <= D) d = mid;
          else c = mid + 1;
        }
        return above + (below_all - P(c - 1));
      };
      // The MAD of rank k is the least occupied distance D with
      // within(D) >= k + 1.  On each side of om the distance grows with the
      // step away from om, and within grows with D, so each side's least
      // qualifying position is found by a search; the lesser of the two
      // sides' distances is attained at an occupied position (within only
      // changes there).  Four searches (ranks k1, k2 x above, below), 128
      // threads each: a round tests the last position of 128 equal chunks
      // of the live span and keeps the first chunk whose test passes, so
      // 65536 positions take three rounds.
      constexpr int kLanes = kFinThreads / 4;
      static_assert(kLanes == 128, "four searches of 128 threads");
      const int combo = tid / kLanes, lt = tid % kLanes;
      const unsigned long long need = ((combo & 1) ? k2 : k1) + 1;
      const bool above = combo < 2;
      const int span_n = above ? kOrdLast + 1 - om : om - kOrdFirst;
      // distance of the i-th position away from m on this side
      auto dist = [&](int i) -> double {
        return above ? val_of_ord(om + i) - m : m - val_of_ord(om - 1 - i);
      };
      int slo = 0, shi = span_n;  // the answer lies in [slo, shi], shi meaning none
      bool found = false;
      if (tid < 12) srch[tid / 4][tid % 4] = kLanes;
      __syncthreads();
      for (int round = 0; round < 3; ++round) {
        const int span = shi - slo;
        const int step = (span + kLanes - 1) / kLanes;
        if (span > 0) {
          int q = slo + (lt + 1) * step - 1;
          q = q < shi - 1 ? q : shi - 1;
          if (slo + lt * step < shi && within(dist(q)) >= need) atomicMin(&srch[round][combo], lt);
        }
        __syncthreads();
        const int c = srch[round][combo];
        if (span > 0) {
          if (c < kLanes) {
            const int nlo = slo + c * step;
            const int nhi = nlo + step < shi ? nlo + step : shi;
            slo = nlo;
            shi = nhi;
            found = true;
          } else if (!found) {
            slo = shi;  // no position on this side qualifies
          }
        }
      }
      // [slo, shi) is now one position (or empty when none qualifies)
      if (lt == 0 && found && slo < span_n) {
        const unsigned long long bits = dbits(__builtin_fabs(dist(slo)));
        atomicMin(&dmin[combo & 1], bits);
      }
      __syncthreads();
      mad = (__longlong_as_double((long long)dmin[0]) + __longlong_as_double((long long)dmin[1])) * 0.5;
    }
  }
  if (tid == 0) {
    moe_audit_stats r;
    r.n = (int64_t)n + (int64_t)n_nan;
    r.n_zero = (int64_t)zero_cnt;
    r.n_nan = (int64_t)n_nan;
    r.median = med;
    r.mad = mad;
    r.sigma_rob = kSigmaRobScale * mad;
    *out = r;
  }
}

// One workgroup per slice histogram (uint32 counts), and the last one for
// the whole tensor's (uint64), all in one launch.
__global__ __launch_bounds__(kFinThreads) void audit_finalize_kernel(uint32_t* __restrict__ hist,
                                                                     unsigned long long* __restrict__ whole,
                                                                     const uint32_t* __restrict__ grp, int slices, moe_audit_stats* __restrict__ out) {
  if ((int)blockIdx.x < slices)
    finalize_one<uint32_t>(hist + (int64_t)blockIdx.x * kBins, grp + (int64_t)blockIdx.x * kGroups, out + blockIdx.x);
  else
    finalize_one<unsigned long long>(whole, nullptr, out + slices);
}

int audit_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

inline size_t up256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// workspace: slice histograms [slices][65536] u32 | tensor histogram [65536]
// u64 | slice group tables [slices][1024] u32
size_t audit_workspace_bytes(int64_t slices) {
  return up256((size_t)slices * kBins * sizeof(uint32_t)) + (size_t)kBins * sizeof(unsigned long long) +
         (size_t)slices * kGroups * sizeof(uint32_t);
}

hipError_t launch_audit(const void* w, int64_t slices, int64_t n, int64_t stride, moe_audit_stats* stats, void* ws,
                        hipStream_t st) {
  uint32_t* hist = static_cast<uint32_t*>(ws);
  char* b = static_cast<char*>(ws) + up256((size_t)slices * kBins * sizeof(uint32_t));
  auto* whole = reinterpret_cast<unsigned long long*>(b);
  b += (size_t)kBins * sizeof(unsigned long long);
  auto* grp = reinterpret_cast<uint32_t*>(b);
  const int64_t n32 = slices * (int64_t)kBins, g32 = slices * (int64_t)kGroups;
  const int64_t cgrid = (n32 + 255) / 256;
  audit_clear_kernel<<<(unsigned)(cgrid < 4096 ? cgrid : 4096), 256, 0, st>>>(hist, n32, whole, grp, g32);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (n > 0) {
    // about eight workgroups per CU over all slices (two are resident at a
    // time: the LDS histogram takes 64 KB), each with at least 64 Ki elements
    int64_t B = (8 * audit_cus() + slices - 1) / slices;
    const int64_t bmax = n / 65536 > 1 ? n / 65536 : 1;
    B = B < bmax ? B : bmax;
    B = B > 0 ? B : 1;
    audit_hist_kernel<<<dim3((unsigned)B, (unsigned)slices), kHistThreads, 0, st>>>(
        static_cast<const uint16_t*>(w), n, stride, hist, whole, grp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  audit_finalize_kernel<<<(unsigned)(slices + 1), kFinThreads, 0, st>>>(hist, whole, grp, (int)slices, stats);
  return hipGetLastError();
}

}  // namespace moe
