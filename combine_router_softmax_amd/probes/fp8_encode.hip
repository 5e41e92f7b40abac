// Check of the library's e4m3 encoder (csrc/fp8_quant.hpp, e4m3_encode2: the
// conversion instruction, values of magnitude <= 2^-10 entered as +0) against
// a bit-level encoder of the OCP e4m3fn format, on every finite float32
// clamped to [-448, 448] (2^32 - 2^24 inputs, each once). A standalone
// program (not part of the library), built beside it; prints
// "tested N mismatches M" and the first mismatching inputs, if any.
//
// Bit-level rule: below 2^-6 the code is the subnormal multiple of 2^-9
// nearest |y| (half to even); above, the float32 mantissa is rounded to 3 bits
// (half to even) with the carry moving into the exponent field (bias 7); the
// sign bit is set for negative values whose code is not zero.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "fp8_quant.hpp"

namespace {

__device__ uint32_t e4m3_bits(float y) {
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    code = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const uint32_t b = __float_as_uint(a);
    code = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return code | (y < 0.f && code != 0u ? 0x80u : 0u);
}

// grid-stride over all 2^32 patterns; every thread's loop ends after
// 2^32 / (grid threads) iterations
__global__ void check(unsigned long long* cnt, uint32_t* first) {
  const uint64_t tid = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint64_t nth = uint64_t(gridDim.x) * blockDim.x;
  unsigned long long tested = 0, bad = 0;
  for (uint64_t i = tid; i < (uint64_t(1) << 32); i += 2 * nth) {
    const uint32_t b0 = uint32_t(i), b1 = uint32_t(i + nth < (uint64_t(1) << 32) ? i + nth : i);
    const float y0 = fminf(fmaxf(__uint_as_float(b0), -448.f), 448.f);
    const float y1 = fminf(fmaxf(__uint_as_float(b1), -448.f), 448.f);
    const uint32_t hw = moe::e4m3_encode2(y0, y1);
    const bool f0 = (b0 & 0x7f800000u) != 0x7f800000u, f1 = (b1 & 0x7f800000u) != 0x7f800000u && b1 != b0;
    const bool m0 = f0 && (hw & 0xffu) != e4m3_bits(y0);
    const bool m1 = f1 && (hw >> 8) != e4m3_bits(y1);
    tested += unsigned(f0) + unsigned(f1);
    if (m0 || m1) {
      bad += unsigned(m0) + unsigned(m1);
      const unsigned long long k = atomicAdd(&cnt[2], 1ull);
      if (k < 8) first[k] = m0 ? b0 : b1;
    }
  }
  atomicAdd(&cnt[0], tested);
  atomicAdd(&cnt[1], bad);
}

}  // namespace

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

int main() {
  unsigned long long* cnt;
  uint32_t* first;
  CHECK(hipMalloc(&cnt, 4 * sizeof(unsigned long long)));
  CHECK(hipMalloc(&first, 8 * sizeof(uint32_t)));
  CHECK(hipMemset(cnt, 0, 4 * sizeof(unsigned long long)));
  CHECK(hipMemset(first, 0, 8 * sizeof(uint32_t)));
  hipLaunchKernelGGL(check, dim3(65536), dim3(256), 0, 0, cnt, first);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  unsigned long long h[4];
  uint32_t f[8];
  CHECK(hipMemcpy(h, cnt, sizeof h, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(f, first, sizeof f, hipMemcpyDeviceToHost));
  printf("tested %llu mismatches %llu\n", h[0], h[1]);
  for (unsigned long long i = 0; i < h[2] && i < 8; ++i) printf("  input %08x\n", f[i]);
  CHECK(hipFree(cnt));
  CHECK(hipFree(first));
  return 0;
}
