/* Exhaustive check of the bf16 quantization's quotient (combine_router_softmax_amd
 * csrc/quant_fp8.hip, e4m3_quant_bf16) against the correctly rounded division.
 *
 * For every finite bf16 block maximum amax >= 0 and every finite bf16 x with
 * |x| <= amax: s = amax / 448 (1 when that is 0); k = 2^64 when s < 2^-64,
 * else 1; r = 1 / (s k); q0 = (x k) r; q = fma(fma(-q0, s k, x k), r, q0).
 * Counts the pairs whose e4m3 code (clamp to +-448, subnormal codes
 * rint(|q| 2^9) below 2^-6, otherwise the mantissa rounded to 3 bits, half
 * to even, zero as 0x00: the rounding of the kernel's conversion
 * instruction) differs from that of x / s, and
 * the pairs with |x / s| >= 2^-10 whose float32 quotients differ. Prints
 * "tested N code_mismatches A quotient_mismatches B". IEEE float32 with
 * subnormals and exact fmaf are assumed (build without fast-math and with
 * -ffp-contract=off). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bf16(uint32_t b) {
  const uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static uint32_t e4m3_code(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = bits_of(a);
    code = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return code | (y < 0.f && code != 0u ? 0x80u : 0u);
}

static float clamp448(float q) { return fminf(fmaxf(q, -448.f), 448.f); }

int main(void) {
  long long tested = 0, bad_code = 0, bad_q = 0;
#pragma omp parallel for reduction(+ : tested, bad_code, bad_q) schedule(dynamic, 64)
  for (uint32_t ab = 0; ab < 0x7F80; ++ab) {
    const float amax = from_bf16(ab);
    float s = amax / 448.f;
    if (!(s > 0.f)) s = 1.f;
    const float k = s < 0x1p-64f ? 0x1p64f : 1.f;
    const float ss = s * k;
    const float r = 1.f / ss;
    for (uint32_t xb = 0; xb < 0x10000; ++xb) {
      if ((xb & 0x7F80) == 0x7F80) continue; /* inf, nan */
      const float x = from_bf16(xb);
      if (fabsf(x) > amax) continue;
      const float xk = x * k;
      const float q0 = xk * r;
      const float q = fmaf(fmaf(-q0, ss, xk), r, q0);
      const float ref = x / s;
      tested++;
      if (e4m3_code(clamp448(ref)) != e4m3_code(clamp448(q))) bad_code++;
      if (fabsf(ref) >= 0x1p-10f && bits_of(ref) != bits_of(q)) bad_q++;
    }
  }
  printf("tested %lld code_mismatches %lld quotient_mismatches %lld\n", tested, bad_code, bad_q);
  return 0;
}
