// Top-K router: softmax over E logits, the K largest by logit, renormalised
// weights (Perplexity, "Lower latency and higher throughput with multi-node
// DeepSeek deployment", section MoE Router).
//
// One wavefront per token. Each lane holds ceil(E/64) logits as 32-bit
// order-preserving integer keys (expert j * 64 + lane), so an unsigned max is
// the highest logit. K rounds select the experts in order: each lane takes its
// best live key (the lowest index among equal keys), a wave-wide max over the
// lanes (DPP row shifts and broadcasts, then a lane read) gives the round's
// key, a ballot finds the lanes holding it, and among several (equal logits)
// the lowest expert index wins. The selection is exact integer comparison, no
// exp involved. Weights use the fp32 exp of (logit - max).
#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kRouteTokensPerBlock = 4;

// Key 0 marks "no expert here / already taken"; every present expert gets a
// key of at least 1, so the K rounds always find K distinct, in-range experts.
// (Only a NaN with a negative sign and an all-ones payload maps to 0 before
// the clamp; NaNs carry no order, so where they land is unspecified.)
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 compare equal
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k > 1u ? k : 1u;
}

__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// max over the wave's 64 lanes: within each row of 16 lanes by right shifts of
// 1, 2, 3, 4 and 8 (lane 15 of a row then holds the row's max), across rows by
// the row-15 and row-31 broadcasts (lane 63 then holds the wave's max); lanes
// a shift reads from outside the row get 0, the identity of an unsigned max
__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t o) { return o > v ? o : v; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xf, 0xf, false)));  // row_shr:1
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xf, 0xf, false)));  // row_shr:2
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x113, 0xf, 0xf, false)));  // row_shr:3
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xf, 0xe, false)));  // row_shr:4
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xf, 0xc, false)));  // row_shr:8
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xa, 0xf, false)));  // row_bcast:15
  v = dpp_max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xc, 0xf, false)));  // row_bcast:31
  return uint32_t(__builtin_amdgcn_readlane(int(v), 63));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = uint32_t(__shfl_xor(int(v), off, kWave));
    v = o < v ? o : v;
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
  uint32_t key[VPL];  // 0: no expert here, or already selected (present experts have keys >= 1)
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * kWave + lane;
    val[j] = e < n_experts ? row[e] : 0.f;
    key[j] = e < n_experts ? order_key(val[j]) : 0u;
  }

  uint32_t mine_key = 0;  // lane k keeps the k-th winner
  int mine_idx = 0;
  for (int k = 0; k < top_k; ++k) {
    // this lane's best live key; the lowest j among equal keys
    uint32_t lb = 0;
    int lj = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (key[j] > lb) {
        lb = key[j];
        lj = j;
      }
    const uint32_t m = wave_max_u32(lb);
    const bool holder = lb == m && m != 0;
    const uint64_t h = __ballot(holder);
    int e;
    if (__popcll(h) == 1) {  // uniform: one lane holds the round's key
      const int hl = __ffsll((unsigned long long)h) - 1;
      e = __builtin_amdgcn_readlane(lj * kWave + lane, hl);
    } else {  // equal logits on several lanes: the lowest expert index
      e = int(wave_min_u32(holder ? uint32_t(lj * kWave + lane) : 0xFFFFFFFFu));
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j * kWave + lane == e) key[j] = 0;
    if (lane == k) {
      mine_key = m;
      mine_idx = e;
    }
  }

  const float vmax = key_value(uint32_t(__builtin_amdgcn_readlane(int(mine_key), 0)));
  const float v = key_value(mine_key);
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
    topk_idx[size_t(t) * top_k + lane] = int32_t(mine_idx);
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
