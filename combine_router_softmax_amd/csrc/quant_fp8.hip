// On-the-fly 1 x 128 fp8 quantization of token rows (the fp8 dispatch payload).
//
// Perplexity, "Lower latency and higher throughput with multi-node DeepSeek
// deployment", section Quantization (activations quantized in 128-element
// vectors); the payload that travels to the experts is fp8 with its scales
// (lehuy.net, "Decoding high-performance EP kernels", section Latency: send
// without asking; Perplexity, "Enabling trillion-parameter models on AWS EFA",
// section Evaluation). Each token row is quantized once, at its source, and
// the dispatch then copies codes and scales.
//
// One pass over HBM: a thread takes 8 consecutive values (one 16-byte bf16
// load), 16 neighbouring threads one 128-value block; the block's largest
// magnitude comes from four lane exchanges, then each thread writes its 8
// codes (8 bytes) and the block's first thread its scale.
#include "fp8_quant.hpp"

namespace moe {
namespace {

constexpr int kQThreads = 256;

// Clamped quotient of a bf16 value v (|v| <= the block's largest magnitude)
// by the block's scale s, formed as q0 = v' r corrected once by a fused
// multiply-add, q = q0 + (v' - q0 s') r, where r = 1 / s' is correctly
// rounded (one division per thread, not eight) and v' = v k, s' = s k with k
// = 2^64 for blocks whose scale is below 2^-64 (exact power-of-two scaling,
// so that the residual stays exact). For every pair of bf16 values this gives
// the correctly rounded quotient wherever it reaches 2^-10 and the same e4m3
// code as the correctly rounded division everywhere (tests/fastdiv_check.c
// runs all 2^30 pairs).
__device__ __forceinline__ float e4m3_quotient_bf16(float v, float k, float ss, float r) {
  const float x = v * k;
  const float q0 = x * r;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, ss, x), r, q0);
  return fminf(fmaxf(q, -kE4m3Max), kE4m3Max);
}

template <typename T>
__global__ __launch_bounds__(kQThreads) void quantize_1x128_kernel(const T* __restrict__ x, int64_t n_blocks,
                                                                  int blocks_per_row, int hidden,
                                                                  uint8_t* __restrict__ xq, float* __restrict__ xs) {
  const int64_t blk = (int64_t(blockIdx.x) * kQThreads + threadIdx.x) >> 4;
  const int part = threadIdx.x & 15;
  // (a block's 16 threads lie in one aligned group of 16 lanes, so they all
  // leave here or all stay, and the exchanges below stay inside the group)
  if (blk >= n_blocks) return;
  const int64_t row = blk / blocks_per_row;
  const int b = int(blk - row * blocks_per_row);
  const size_t off = size_t(row) * hidden + size_t(b) * 128 + size_t(part) * 8;
  float v[8];
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(x + off);
    const float4 c = *reinterpret_cast<const float4*>(x + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float s = e4m3_block_scale(m);
  uint32_t lo = 0, hi = 0;
  if constexpr (sizeof(T) == 2) {
    const float k = s < 0x1p-64f ? 0x1p64f : 1.f;
    const float ss = s * k;
    const float r = 1.f / ss;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = e4m3_quotient_bf16(v[i], k, ss, r);
    lo = e4m3_encode2(q[0], q[1]) | e4m3_encode2(q[2], q[3]) << 16;
    hi = e4m3_encode2(q[4], q[5]) | e4m3_encode2(q[6], q[7]) << 16;
  } else {  // float32 inputs: the correctly rounded division of each value
    lo = e4m3_quant4(v[0], v[1], v[2], v[3], s);
    hi = e4m3_quant4(v[4], v[5], v[6], v[7], s);
  }
  *reinterpret_cast<uint2*>(xq + off) = make_uint2(lo, hi);
  if (part == 0) xs[blk] = s;
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API moe_status_t moe_quantize_1x128(const void* x, moe_dtype_t dt, int64_t n_rows, int hidden, uint8_t* xq,
                                        float* xs, hipStream_t stream) {
  if (n_rows < 0 || hidden < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16 && dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (hidden % 128) return MOE_ERR_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  if (!x || !xq || !xs || !aligned16(x) || (reinterpret_cast<uintptr_t>(xq) & 7u) ||
      (reinterpret_cast<uintptr_t>(xs) & 3u))
    return MOE_ERR_INVALID_ARG;
  const int bpr = hidden / 128;
  const int64_t n_blocks = n_rows * bpr;
  const int64_t groups = (n_blocks * 16 + kQThreads - 1) / kQThreads;
  if (groups >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid{unsigned(groups)}, block{unsigned(kQThreads)};
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(quantize_1x128_kernel<uint16_t>, grid, block, 0, stream, static_cast<const uint16_t*>(x),
                       n_blocks, bpr, hidden, xq, xs);
  else
    hipLaunchKernelGGL(quantize_1x128_kernel<float>, grid, block, 0, stream, static_cast<const float*>(x), n_blocks,
                       bpr, hidden, xq, xs);
  return launch_status();
}
