// Top-K router: softmax over E logits, the K largest by logit, renormalised
// weights (Perplexity, "Lower latency and higher throughput with multi-node
// DeepSeek deployment", section MoE Router).
//
// One wavefront per token. Each lane holds ceil(E/64) logits as 64-bit keys
// (order-preserving integer image of the fp32 logit in the high word, the
// complement of the expert index in the low word), so one unsigned max picks
// the highest logit and, among equal logits, the lowest index. K rounds of a
// wave-wide max (xor butterfly) select the experts in order; the selection is
// exact integer comparison, no exp involved. Weights use the fp32 exp of
// (logit - max).
#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kRouteTokensPerBlock = 4;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor((unsigned long long)v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(kWave * kRouteTokensPerBlock) void route_topk_kernel(
    const float* __restrict__ logits, int n_tokens, int n_experts, int top_k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteTokensPerBlock + (threadIdx.x / kWave);
  if (t >= n_tokens) return;  // uniform per wave
  const float* row = logits + size_t(t) * n_experts;

  float val[VPL];
  uint64_t cand[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * kWave + lane;
    if (e < n_experts) {
      val[j] = row[e];
      cand[j] = (uint64_t(order_key(val[j])) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(e));
    } else {
      val[j] = 0.f;
      cand[j] = 0;  // below every real key (a real key's low word is > 0)
    }
  }

  uint64_t mine = 0;  // lane k keeps the k-th winner
  for (int k = 0; k < top_k; ++k) {
    uint64_t best = cand[0];
#pragma unroll
    for (int j = 1; j < VPL; ++j) best = cand[j] > best ? cand[j] : best;
    best = wave_max_u64(best);
    const int e = int(0xFFFFFFFFu - uint32_t(best));
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j * kWave + lane == e) cand[j] = 0;
    if (lane == k) mine = best;
  }

  const float vmax = key_value(uint32_t((unsigned long long)__shfl((unsigned long long)mine, 0, kWave) >> 32));
  const float v = key_value(uint32_t(mine >> 32));
  const float ex = lane < top_k ? expf(v - vmax) : 0.f;
  float denom;
  if (renorm) {
    denom = wave_sum_f32(ex);
  } else {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j * kWave + lane < n_experts) part += expf(val[j] - vmax);
    denom = wave_sum_f32(part);
  }
  if (lane < top_k) {
    topk_idx[size_t(t) * top_k + lane] = int32_t(0xFFFFFFFFu - uint32_t(mine));
    topk_w[size_t(t) * top_k + lane] = ex / denom;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

MOE_API moe_status_t moe_route_topk(const float* logits, int n_tokens, int n_experts, int top_k, int renormalize,
                                    int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  if (n_tokens < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts) return MOE_ERR_INVALID_ARG;
  if (n_experts > 1024 || top_k > 16) return MOE_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if ((size_t)n_tokens * (size_t)n_experts >= (size_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid((n_tokens + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock);
  const dim3 block(kWave * kRouteTokensPerBlock);
  const int vpl = (n_experts + kWave - 1) / kWave;
#define MOE_ROUTE_LAUNCH(V) \
  hipLaunchKernelGGL(route_topk_kernel<V>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, \
                     renormalize, topk_idx, topk_w)
  if (vpl <= 1) MOE_ROUTE_LAUNCH(1);
  else if (vpl <= 2) MOE_ROUTE_LAUNCH(2);
  else if (vpl <= 4) MOE_ROUTE_LAUNCH(4);
  else if (vpl <= 8) MOE_ROUTE_LAUNCH(8);
  else MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
  return launch_status();
}
