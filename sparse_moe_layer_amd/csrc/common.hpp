// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }  // round to nearest even

// 1 / (1 + e^-z) with the hardware reciprocal (v_rcp_f32, about 1 ulp): the
// argument is >= 1 (or +inf, whose reciprocal is 0), so no scaling is needed,
// and it replaces the ten-instruction IEEE division in every epilogue.
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }

// 16-byte global load / store helpers (addresses must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// 16-byte accesses marked non-temporal: data read once (streamed expert
// weights) or written once and read back only by a later launch.
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Eight OCP e4m3fn codes (two dwords) times one fp32 scale -> eight bf16.
// gfx950's v_cvt_pk_f32_fp8 decodes the OCP E4M3FN format.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 codes, float scale) {
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(codes[h], false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(codes[h], true);
    bf16x2 pa = {f2bf(a.x * scale), f2bf(a.y * scale)};
    bf16x2 pb = {f2bf(b.x * scale), f2bf(b.y * scale)};
    out[2 * h] = __builtin_bit_cast(uint32_t, pa);
    out[2 * h + 1] = __builtin_bit_cast(uint32_t, pb);
  }
  return out;
}

// Eight OCP e4m3fn codes -> eight bf16, exactly (every e4m3fn value is a
// bf16 value): gfx950's scaled conversion at scale 1.0, two codes per
// instruction.  (Its scale operand contributes only its power-of-two
// exponent, so a block scale cannot be folded in here.)
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8_exact(u32x2 codes) {
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    out[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[h], 1.0f, false));
    out[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[h], 1.0f, true));
  }
  return out;
}

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

}  // namespace moe
