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

// IEEE binary64 -> FP8 E4M3 (OCP: sign, 4 exponent bits with bias 7, 3
// mantissa bits, exponent 0 subnormal, S.1111.111 NaN, largest finite 448),
// round to nearest even in one rounding, sign kept; magnitudes from 448 up
// (and infinities) saturate to 448, NaN gives 0x7F.
__device__ __forceinline__ uint8_t f64_to_e4m3(double x) {
  const uint8_t sign = (uint8_t)((__builtin_bit_cast(uint64_t, x) >> 56) & 0x80u);
  const double a = __builtin_fabs(x);
  if (a != a) return 0x7Fu;
  if (a >= 448.0) return sign | 0x7Eu;
  if (a == 0.0) return sign;
  int e2;
  (void)__builtin_frexp(a, &e2);  // a in [2^(e2-1), 2^e2)
  int e = e2 - 1;
  if (e < -6) {
    // subnormal grid m 2^-9; m = 8 is the smallest normal, code 0x08 itself
    return sign | (uint8_t)__builtin_rint(__builtin_ldexp(a, 9));
  }
  double m = __builtin_rint(__builtin_ldexp(a, 3 - e));  // in [8, 16]
  if (m == 16.0) {
    m = 8.0;
    ++e;
  }
  return sign | (uint8_t)((e + 7) << 3) | (uint8_t)((int)m - 8);
}

__device__ __forceinline__ double e4m3_to_f64(uint8_t c) {
  const int e = (c >> 3) & 0xF, m = c & 7;
  if ((c & 0x7F) == 0x7F) return __builtin_nan("");
  const double mag = e == 0 ? __builtin_ldexp((double)m, -9) : __builtin_ldexp((double)(8 + m), e - 10);
  return (c & 0x80) ? -mag : mag;
}

// A group's stored (scale, zero) pair and the values the codes are taken
// against.  MB = 4: two fp16, scale in the low half; MB = 2: two FP8 E4M3
// bytes, scale in the low byte.  A group holding NaN stores NaN for both.
template <int MB>
__device__ __forceinline__ uint32_t encode_sz(double s, double z, double& sd, double& zd) {
  if constexpr (MB == 4) {
    const uint16_t sb = f64_to_f16_bits(s), zb = f64_to_f16_bits(z);
    sd = f16_bits_to_f64(sb);
    zd = f16_bits_to_f64(zb);
    return (uint32_t)sb | ((uint32_t)zb << 16);
  } else {
    const uint8_t sb = f64_to_e4m3(s), zb = f64_to_e4m3(z);
    sd = e4m3_to_f64(sb);
    zd = e4m3_to_f64(zb);
    return (uint32_t)sb | ((uint32_t)zb << 8);
  }
}
template <int MB>
__device__ __forceinline__ uint32_t nan_sz() {
  return MB == 4 ? 0x7e007e00u : 0x7F7Fu;
}
// store one pair at byte address p (MB bytes)
template <int MB>
__device__ __forceinline__ void store_sz(uint8_t* p, uint32_t pair) {
  if constexpr (MB == 4)
    *(uint32_t*)p = pair;
  else
    *(uint16_t*)p = (uint16_t)pair;
}

}  // namespace oscar
