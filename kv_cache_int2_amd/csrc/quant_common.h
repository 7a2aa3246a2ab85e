// Device helpers of the INT2 quantiser, shared by the write kernels and the
// fused decode-step front kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

// IEEE binary64 -> binary16, round to nearest even (single rounding).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) return sign | (a > 0x7ff0000000000000ull ? 0x7e00u : 0x7c00u);
  if (a == 0) return sign;
  int e = (int)(a >> 52) - 1023;
  uint64_t m = a & 0x000fffffffffffffull;
  if (e == -1023) {
    return sign;  // binary64 subnormal: far below half the smallest binary16 subnormal
  }
  m |= 1ull << 52;
  if (e >= -14) {
    uint64_t mant = m >> 42;
    const uint64_t rem = m & ((1ull << 42) - 1);
    const uint64_t half = 1ull << 41;
    if (rem > half || (rem == half && (mant & 1))) ++mant;
    if (mant == 2048) {
      mant = 1024;
      ++e;
    }
    if (e > 15) return sign | 0x7c00u;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(mant & 0x3ffu);
  }
  const int shift = 28 - e;  // >= 43
  if (shift >= 64) return sign;
  uint64_t mant = m >> shift;
  const uint64_t rem = m & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (mant & 1))) ++mant;
  return sign | (uint16_t)mant;
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

}  // namespace oscar
