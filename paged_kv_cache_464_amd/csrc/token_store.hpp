// Device helpers shared by the reshape-and-cache scatter and the fused decode
// step: the fp8 E4M3FN and int8 encoders of a new token's K/V (youngju.dev
// "KV cache and paged attention", section "KV 양자화: FP8과 INT8": one byte
// per element, int8 with a scale and a zero point).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace pa {

// OCP E4M3FN encode of an fp32 value: NaN -> 0x7F, |y| >= 448 -> +-448
// (saturation), otherwise round to nearest, ties to even mantissa code.
// Integer arithmetic on the fp32 bit pattern, so the result is exact.
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;        // >= 448.0f: saturate
  if (a < 0x3C800000u) {                            // < 2^-6: spacing 2^-9
    const float q = rintf(__uint_as_float(a) * 512.0f);  // exact scale, then RNE
    return sign | static_cast<uint32_t>(q);         // q in [0, 8]; 8 is 2^-6 (code 8)
  }
  const uint32_t e = (a >> 23) - 127u + 7u;         // biased e4m3 exponent, 1..15
  uint32_t keep = ((a >> 20) & 0x7u) | (e << 3);    // code before rounding
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;  // carry into exponent is correct
  return sign | keep;
}

// int8 code of y = x * inv_scale: y rounded to the nearest integer (ties to
// even), plus the zero point, saturated to [-128, 127]; NaN gives the zero
// point and infinities saturate.  Returned as the stored byte c + 128.
__device__ inline uint32_t i8_encode_stored(float y, float zero) {
  float r = rintf(y);
  // NaN test on the bit pattern: it must hold where the compiler may assume
  // that no value is NaN (the decode kernels are built so).
  r = (__float_as_uint(r) & 0x7FFFFFFFu) > 0x7F800000u ? 0.0f : r;
  const float c = fminf(fmaxf(r + zero, -128.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int>(c) + 128);
}

// The stored byte of y = x * inv_scale in a pool of the given one-byte kind.
template <int KIND>
__device__ inline uint32_t encode_byte(float y, float zero) {
  if constexpr (KIND == kI8) return i8_encode_stored(y, zero);
  (void)zero;
  return e4m3_encode(y);
}

__device__ inline float half_bits_to_float(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

}  // namespace pa
