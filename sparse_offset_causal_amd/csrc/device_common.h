// Device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace soc {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16_t))));
typedef bf16_t bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16_t))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));

#define SOC_NEG_INF (-__builtin_inff())

// Cache policy operand of a buffer load for data read once per call (the nt bit of gfx950's
// cache policy): whole lines a wave reads in one instruction and never asks for again.  It is
// not used where a wave reads part of a line and relies on the cache for the rest of it (the
// MFMA-layout K loads of decode), nor where other workgroups re-read the same tiles (prefill).
constexpr int kLoadReadOnce = 2;

// Raw hardware 2^x (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 32x32x16 bf16 MFMA, fp32 accumulate.  Lane l holds A[l%32][8*(l/32)+0..7],
// B[8*(l/32)+0..7][l%32]; D[i][j] for j = l%32, i = 8*(v/4) + 4*(l/32) + v%4 (v = 0..15).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// bf16 -> float is exact: the bf16 bits are the top half of the float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Lanes l and l^32 (the two halves of a wave64) exchange a value with gfx950's
// v_permlane32_swap; with both operands = x the pair comes back as {x[l & 31], x[l | 32]},
// so symmetric combinations of the pair give the same result in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

// Order-preserving map of doubles to unsigned 64-bit keys (ascending).
__device__ __forceinline__ uint64_t f64_order_key(double x) {
  uint64_t b = __builtin_bit_cast(uint64_t, x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double f64_from_order_key(uint64_t k) {
  uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __builtin_bit_cast(double, b);
}

}  // namespace soc
