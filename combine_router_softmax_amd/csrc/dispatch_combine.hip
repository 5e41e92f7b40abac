// Dispatch (token rows -> expert-grouped rows) and combine (expert rows ->
// router-weighted sum in token order).
//
// Both are pure HBM streams: one wavefront per token, 16-byte vector loads and
// stores, every lane moving consecutive 16-byte pieces of the row so a wave
// instruction covers 1 KiB of contiguous memory. Dispatch reads each token row
// once and writes it to each of its slots (lehuy.net, "Decoding
// high-performance EP kernels", section Throughput > Dispatch). Combine reads
// the up-to-K expert rows of a token (and the shared-expert row), accumulates
// w * y in fp32 in k order and rounds once (same page, section Combine; the sum
// over this GPU's experts is formed at the sender, Perplexity, "Enabling
// trillion-parameter models on AWS EFA", section Evaluation).
#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;
constexpr int kMaxK = 16;

template <int U>
__global__ __launch_bounds__(kWave * kTokensPerBlock) void dispatch_kernel(
    const uint4* __restrict__ x, int n_tokens, int row_vecs, int top_k, const int32_t* __restrict__ row_of,
    int64_t n_rows, uint4* __restrict__ xe) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokensPerBlock + threadIdx.x / kWave;
  if (t >= n_tokens) return;
  int my_row = -1;
  if (lane < top_k) my_row = row_of[size_t(t) * top_k + lane];
  const bool ok = lane < top_k && my_row >= 0 && int64_t(my_row) < n_rows;
  const uint64_t mask = __ballot(ok);
  if (mask == 0) return;
  const uint4* src = x + size_t(t) * row_vecs;
  for (int c0 = 0; c0 < row_vecs; c0 += kWave * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c < row_vecs) v[u] = src[c];
    }
    uint64_t m = mask;
    while (m) {
      const int k = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int r = __shfl(my_row, k, kWave);
      uint4* dst = xe + size_t(r) * row_vecs;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row_vecs) dst[c] = v[u];
      }
    }
  }
}

// 16-byte piece <-> floats
template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 store(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static uint4 store(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

template <typename T, int KMAX, int U>
__global__ __launch_bounds__(kWave * kTokensPerBlock) void combine_kernel(
    const uint4* __restrict__ ye, int64_t n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
    int n_tokens, int top_k, int row_vecs, const uint4* __restrict__ shared_y, int self_lo, int self_hi,
    uint4* __restrict__ out) {
  constexpr int EPV = Vec<T>::N;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kTokensPerBlock + threadIdx.x / kWave;
  if (t >= n_tokens) return;
  int my_row = -1;
  float my_w = 0.f;
  if (lane < top_k) {
    my_row = row_of[size_t(t) * top_k + lane];
    my_w = topk_w[size_t(t) * top_k + lane];
  }
  const bool ok = lane < top_k && my_row >= 0 && int64_t(my_row) < n_rows;
  const uint64_t mask = __ballot(ok);
  const bool in_self = shared_y != nullptr && t >= self_lo && t < self_hi;
  if (mask == 0 && !in_self) return;

  // compact the kept (row, weight) pairs, k ascending, into uniform registers
  int rows[KMAX];
  float ws[KMAX];
  int nk = 0;
  {
    uint64_t m = mask;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      rows[i] = 0;
      ws[i] = 0.f;
      if (m) {
        const int k = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        rows[i] = __shfl(my_row, k, kWave);
        ws[i] = __shfl(my_w, k, kWave);
        nk = i + 1;
      }
    }
  }
  const uint4* sy = in_self ? shared_y + size_t(t - self_lo) * row_vecs : nullptr;
  uint4* dst = out + size_t(t) * row_vecs;

  for (int c0 = 0; c0 < row_vecs; c0 += kWave * U) {
    uint4 v[KMAX][U];
    uint4 vs[U];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < nk) {
        const uint4* src = ye + size_t(rows[i]) * row_vecs;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * kWave + lane;
          if (c < row_vecs) v[i][u] = src[c];
        }
      }
    }
    if (in_self) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave + lane;
        if (c < row_vecs) vs[u] = sy[c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kWave + lane;
      if (c >= row_vecs) continue;
      float acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        if (i < nk) {
          float f[EPV];
          Vec<T>::load(v[i][u], f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[e] = fmaf(ws[i], f[e], acc[e]);
        }
      }
      if (in_self) {
        float f[EPV];
        Vec<T>::load(vs[u], f);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += f[e];
      }
      dst[c] = Vec<T>::store(acc);
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

static bool row_dtype_ok(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

MOE_API moe_status_t moe_dispatch(const void* x, moe_dtype_t dt, int n_tokens, int hidden, int top_k,
                                  const int32_t* row_of, int64_t n_rows, void* xe, hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || top_k < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!row_dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  const size_t row_bytes = size_t(hidden) * dtype_size(dt);
  if (row_bytes % 16) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_rows == 0) return MOE_OK;
  if (!x || !row_of || !xe || !aligned16(x) || !aligned16(xe)) return MOE_ERR_INVALID_ARG;
  const int row_vecs = int(row_bytes / 16);
  const dim3 grid((n_tokens + kTokensPerBlock - 1) / kTokensPerBlock), block(kWave * kTokensPerBlock);
  hipLaunchKernelGGL(dispatch_kernel<8>, grid, block, 0, stream, static_cast<const uint4*>(x), n_tokens, row_vecs,
                     top_k, row_of, n_rows, static_cast<uint4*>(xe));
  return launch_status();
}

template <typename T, int KMAX>
static void launch_combine(dim3 grid, dim3 block, hipStream_t stream, const void* ye, int64_t n_rows,
                           const int32_t* row_of, const float* topk_w, int n_tokens, int top_k, int row_vecs,
                           const void* shared_y, int self_lo, int self_hi, void* out) {
  constexpr int U = KMAX > 8 ? 1 : 2;
  hipLaunchKernelGGL((combine_kernel<T, KMAX, U>), grid, block, 0, stream, static_cast<const uint4*>(ye), n_rows,
                     row_of, topk_w, n_tokens, top_k, row_vecs, static_cast<const uint4*>(shared_y), self_lo,
                     self_hi, static_cast<uint4*>(out));
}

MOE_API moe_status_t moe_combine(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                                 const float* topk_w, int n_tokens, int top_k, int hidden, const void* shared_y,
                                 int self_lo, int self_hi, void* out, hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || top_k < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!row_dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  const size_t row_bytes = size_t(hidden) * dtype_size(dt);
  if (row_bytes % 16) return MOE_ERR_INVALID_ARG;
  if (shared_y && (self_lo < 0 || self_hi < self_lo || self_hi > n_tokens)) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  if (!row_of || !topk_w || !out || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (n_rows > 0 && (!ye || !aligned16(ye))) return MOE_ERR_INVALID_ARG;
  if (shared_y && !aligned16(shared_y)) return MOE_ERR_INVALID_ARG;
  const int row_vecs = int(row_bytes / 16);
  const dim3 grid((n_tokens + kTokensPerBlock - 1) / kTokensPerBlock), block(kWave * kTokensPerBlock);
  const int kmax = top_k <= 2 ? 2 : top_k <= 4 ? 4 : top_k <= 8 ? 8 : 16;
#define MOE_COMBINE(T, KM)                                                                                    \
  launch_combine<T, KM>(grid, block, stream, ye, n_rows, row_of, topk_w, n_tokens, top_k, row_vecs, shared_y, \
                        self_lo, self_hi, out)
  if (dt == MOE_F32) {
    if (kmax == 2) MOE_COMBINE(float, 2);
    else if (kmax == 4) MOE_COMBINE(float, 4);
    else if (kmax == 8) MOE_COMBINE(float, 8);
    else MOE_COMBINE(float, 16);
  } else {
    if (kmax == 2) MOE_COMBINE(uint16_t, 2);
    else if (kmax == 4) MOE_COMBINE(uint16_t, 4);
    else if (kmax == 8) MOE_COMBINE(uint16_t, 8);
    else MOE_COMBINE(uint16_t, 16);
  }
#undef MOE_COMBINE
  return launch_status();
}
