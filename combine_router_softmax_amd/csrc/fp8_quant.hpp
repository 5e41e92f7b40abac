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

// e4m3fn codes of a and b, |a|, |b| <= 448 (OCP 8-bit floating point,
// E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits), rounded to
// nearest, ties to the even code (subnormal multiples of 2^-9 below 2^-6):
// code(a) | code(b) << 8. The conversion instruction rounds exactly so (a
// probe compared it with a bit-level encoder on every finite float32 in
// [-448, 448]) except that a negative value rounding to zero gives the code
// of -0; values of magnitude <= 2^-10, which round to zero, enter as +0 so
// that the code of a zero is 0x00.
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
  const float za = fabsf(a) <= 0x1p-10f ? 0.f : a;
  const float zb = fabsf(b) <= 0x1p-10f ? 0.f : b;
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(za, zb, 0, false)) & 0xffffu;
}

__device__ __forceinline__ uint32_t e4m3_encode(float y) { return e4m3_encode2(y, y) & 0xffu; }

// Scale of a block from its largest magnitude.
__device__ __forceinline__ float e4m3_block_scale(float amax) {
  const float s = amax / kE4m3Max;
  return s > 0.f ? s : 1.f;
}

// Code of v in a block of scale s.
__device__ __forceinline__ float e4m3_clamped_quotient(float v, float s) {
  return fminf(fmaxf(v / s, -kE4m3Max), kE4m3Max);
}
__device__ __forceinline__ uint32_t e4m3_quant(float v, float s) { return e4m3_encode(e4m3_clamped_quotient(v, s)); }

// Codes of four values of a block, packed (first value in the low byte).
__device__ __forceinline__ uint32_t e4m3_quant4(float v0, float v1, float v2, float v3, float s) {
  return e4m3_encode2(e4m3_clamped_quotient(v0, s), e4m3_clamped_quotient(v1, s)) |
         e4m3_encode2(e4m3_clamped_quotient(v2, s), e4m3_clamped_quotient(v3, s)) << 16;
}

}  // namespace moe
