// E4M3 (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, S.1111.111 = NaN, largest finite 448) on the device.  gfx950's
// f8f6f4 matrix instructions read this format as format 0.
#pragma once

#include "common.h"

namespace moe {

constexpr float kF8Max = 448.0f;  // largest finite E4M3 value

// |v| <= 448 -> E4M3 code, nearest with ties to even.  Below 2^-6 the code
// is the number of 2^-9 steps.  Above, the float32 bit pattern already holds
// the E4M3 fields: keep its top 3 mantissa bits, round the 20 dropped ones to
// nearest even (a carry out of the mantissa moves to the next binade by
// itself) and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u)  // 2^-6
    code = (uint32_t)rintf(__fmul_rn(__uint_as_float(a), 512.0f));
  else
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  return code | sign;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e4 = (c >> 3) & 15u, m3 = c & 7u;
  const float mag = e4 == 0 ? ldexpf((float)m3, -9) : ldexpf((float)(8u + m3), (int)e4 - 10);
  return (c & 0x80u) ? -mag : mag;
}

// The decoded value of a finite code in units of 2^-9 (every E4M3 value is
// an integer multiple of 2^-9, at most 448 * 2^9 = 229376 in magnitude).
__device__ __forceinline__ int e4m3_units(uint32_t c) {
  const uint32_t e4 = (c >> 3) & 15u, m3 = c & 7u;
  const int mag = e4 == 0 ? (int)m3 : (int)((8u + m3) << (e4 - 1u));
  return (c & 0x80u) ? -mag : mag;
}

}  // namespace moe
