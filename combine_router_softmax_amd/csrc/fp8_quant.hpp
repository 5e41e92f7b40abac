// 1 x 128 fp8 quantization of activations (internal header).
//
// Perplexity, "Lower latency and higher throughput with multi-node DeepSeek
// deployment", section Quantization: activations are quantized on the fly
// with one scale per 128-element vector (and the SiLU step quantizes its
// output the same way). Rule used here, for a block v[0..127]:
//   s = fp32(max |v|) / 448, and s = 1 where that quotient is 0;
//   code[i] = RNE(clamp(fp32(v[i]) / s, -448, 448)) in OCP e4m3fn,
// with correctly rounded fp32 division and the code of a zero written as 0x00.
// NaN inputs give unspecified (finite) codes.
#pragma once

#include "moe_common.hpp"

namespace moe {

constexpr float kE4m3Max = 448.f;  // largest finite OCP e4m3fn magnitude

// e4m3fn code of y, |y| <= 448 (OCP 8-bit floating point, E4M3: sign, 4
// exponent bits with bias 7, 3 mantissa bits), rounded to nearest, ties to
// the even code. Below 2^-6 the codes are subnormal multiples of 2^-9; above,
// the fp32 mantissa is cut to 3 bits with round-half-even and a carry moves
// into the exponent field.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    code = uint32_t(__builtin_rintf(a * 512.f));  // 0..8; 8 is 2^-6, the first normal code
  } else {
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7ffffu + ((b >> 20) & 1u);
    code = (r >> 20) - ((127u - 7u) << 3);
  }
  return code | (y < 0.f && code != 0u ? 0x80u : 0u);
}

// Scale of a block from its largest magnitude.
__device__ __forceinline__ float e4m3_block_scale(float amax) {
  const float s = amax / kE4m3Max;
  return s > 0.f ? s : 1.f;
}

// Code of v in a block of scale s.
__device__ __forceinline__ uint32_t e4m3_quant(float v, float s) {
  const float y = fminf(fmaxf(v / s, -kE4m3Max), kE4m3Max);
  return e4m3_encode(y);
}

}  // namespace moe
