// E4M3 (OCP FP8) encoding of the 8-bit cache, shared by the append kernel and
// the decode kernel's fused append, so both store the same codes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {
namespace codec {

// E4M3 code of a binary32 value: nearest, ties to the even code, magnitudes
// of 448 and more clamped to 448 (the largest code, 0x7E), NaN kept as NaN.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |y| >= 448
  if (a < 0x3C800000u) {                      // |y| < 2^-6: subnormal codes m * 2^-9
    const float m = __builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
    return sign | uint32_t(m);                // m = 8 is the smallest normal, 0x08
  }
  // normal: biased exponent (e - 127) + 7 in 1..15, three mantissa bits kept
  uint32_t code = ((a >> 23) - 120u) << 3 | ((a >> 20) & 7u);
  const uint32_t rest = a & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ++code;  // a carry moves the exponent
  return sign | code;  // < 448 keeps the code at or below 0x7E
}

// x / scale rounded to binary32: the binary64 quotient of two binary32 values
// rounds to the correctly rounded binary32 quotient.
__device__ __forceinline__ uint32_t quantize_bf16(uint32_t bits16, float scale) {
  const float x = __uint_as_float(bits16 << 16);
  return e4m3_code(float(double(x) / double(scale)));
}

// Eight bf16 values (one 16-byte chunk) -> eight codes (8 bytes).
__device__ __forceinline__ uint2 quantize_chunk(uint4 in, float scale) {
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t p = w[2 * k], q = w[2 * k + 1];  // elements 4k .. 4k+3
    out[k] = quantize_bf16(p & 0xFFFFu, scale) | quantize_bf16(p >> 16, scale) << 8 |
             quantize_bf16(q & 0xFFFFu, scale) << 16 | quantize_bf16(q >> 16, scale) << 24;
  }
  return make_uint2(out[0], out[1]);
}

}  // namespace codec
}  // namespace pa
