// Nearest OCP FP8 E4M3FN code of an fp32 value, ties to even, saturating at
// +-448, NaN kept (with its sign).  Magnitudes below 2^-6 are multiples of
// 2^-9 (subnormal codes m = 0..8, where m = 8 is the smallest normal); above,
// q = 2^E (1 + f) keeps three fraction bits.  Both are a round-to-nearest-
// even of |q| scaled by a power of two (exact in fp32), so rintf does the
// rounding.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mfa {

__device__ __forceinline__ uint8_t e4m3fn_encode(float q) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  if (q != q) return (uint8_t)(sign | 0x7Fu);
  const float a = fminf(fabsf(q), 448.f);
  uint32_t mag;
  if (a < 0.015625f) {                       // below 2^-6: steps of 2^-9
    mag = (uint32_t)__builtin_rintf(a * 512.f);   // 0 .. 8 (8 = smallest normal)
  } else {
    const int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xFF) - 127;   // -6 .. 8
    const float m = __builtin_rintf(a * __builtin_ldexpf(8.f, -e));            // 8 .. 16
    uint32_t mi = (uint32_t)m;
    int eb = e + 7;
    if (mi == 16) {
      mi = 8;
      ++eb;
    }
    mag = ((uint32_t)eb << 3) | (mi - 8);
  }
  return (uint8_t)(sign | mag);
}


}  // namespace mfa
