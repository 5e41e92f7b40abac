// Dispatch (token rows -> expert-grouped rows) and combine (expert rows ->
// router-weighted sum in token order).
//
// Both are pure HBM streams of 16-byte vector loads and stores: a workgroup
// covers 4 KiB of one token row (consecutive lanes, consecutive 16-byte
// pieces, so a wave instruction covers 1 KiB of contiguous memory), and a row
// of 7168 bf16 spreads over 4 workgroups, which gives thousands of independent
// workgroups to hide HBM latency. Dispatch reads each token row
// once and writes it to each of its slots (lehuy.net, "Decoding
// high-performance EP kernels", section Throughput > Dispatch). Combine reads
// the up-to-K expert rows of a token (and the shared-expert row), accumulates
// w * y in fp32 in k order and rounds once (same page, section Combine; the sum
// over this GPU's experts is formed at the sender, Perplexity, "Enabling
// trillion-parameter models on AWS EFA", section Evaluation).
#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kVecThreads = 256;  // one 16-byte piece per thread, 4 KiB of a row per workgroup
constexpr int kMaxK = 16;

// Workgroup b handles 16-byte pieces [chunk * 256, chunk * 256 + 256) of token
// t = b / n_chunks: the token's slots are uniform per workgroup (scalar loads),
// every thread loads one piece and stores it to each slot.
template <int KMAX>
__global__ __launch_bounds__(kVecThreads) void dispatch_kernel(const uint4* __restrict__ x, int row_vecs, int n_chunks,
                                                                int top_k, const int32_t* __restrict__ row_of,
                                                                int64_t n_rows, uint4* __restrict__ xe) {
  const int t = blockIdx.x / n_chunks;
  const int c = (blockIdx.x - t * n_chunks) * kVecThreads + threadIdx.x;
  const int32_t* ro = row_of + size_t(t) * top_k;
  int r[KMAX];
  bool any = false;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < top_k ? ro[k] : -1;
    if (r[k] >= n_rows) r[k] = -1;
    any |= r[k] >= 0;
  }
  if (!any || c >= row_vecs) return;
  const uint4 v = x[size_t(t) * row_vecs + c];
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (r[k] >= 0) xe[size_t(r[k]) * row_vecs + c] = v;
}

// Row-wise dispatch into the 16-row blocked layout: a unit of work is one
// group of 16 output rows x 128 columns (four 1 KiB blocks, contiguous in xe).
// Wave w reads rows 4w..4w+3 of the group, 256 contiguous bytes each, and
// every lane stores its 16 bytes at their blocked position, so the workgroup
// writes 4 KiB of contiguous memory. Persistent workgroups walk the units up
// to the device-side row count.
constexpr int kBlkCols = 128;  // columns per unit
__global__ __launch_bounds__(kVecThreads) void dispatch_blocked_kernel(const uint4* __restrict__ x, int hidden,
                                                                        int n_tokens,
                                                                        const int32_t* __restrict__ row_token,
                                                                        int64_t n_rows,
                                                                        const int32_t* __restrict__ n_used,
                                                                        uint16_t* __restrict__ xe) {
  const int64_t rows = n_used ? min<int64_t>(max(n_used[0], 0), n_rows) : n_rows;
  const int ncu = (hidden + kBlkCols - 1) / kBlkCols;  // column units per row group
  const int64_t units = (rows + 15) / 16 * ncu;
  const int tid = threadIdx.x;
  const int ri = tid >> 4;         // row inside the group (wave w: rows 4w..4w+3)
  const int piece = tid & 15;      // 16-byte piece inside the unit's 256 bytes of the row
  const int row_vecs = hidden / 8;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t g = u / ncu;
    const int cu = int(u - g * ncu);
    const int64_t r = g * 16 + ri;
    const int col = cu * kBlkCols + piece * 8;
    if (r >= rows || col >= hidden) continue;
    const int t = row_token[r];
    if (t < 0 || t >= n_tokens) continue;  // a hole (or an invalid entry): not written
    const uint4 v = x[size_t(t) * row_vecs + col / 8];
    const size_t off = (size_t(g) * (hidden >> 5) + (col >> 5)) * 512 + size_t(ri) * 32 + (col & 31);
    *reinterpret_cast<uint4*>(xe + off) = v;
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

// Same decomposition as dispatch: each thread owns one 16-byte piece of the
// output row and sums the token's kept expert rows in k order (all K loads in
// flight at once), plus the shared-expert row for the GPU's own tokens.
template <typename T, int KMAX>
__global__ __launch_bounds__(kVecThreads) void combine_kernel(
    const uint4* __restrict__ ye, int64_t n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
    int top_k, int row_vecs, int n_chunks, const uint4* __restrict__ shared_y, int self_lo, int self_hi,
    uint4* __restrict__ out) {
  constexpr int EPV = Vec<T>::N;
  const int t = blockIdx.x / n_chunks;
  const int c = (blockIdx.x - t * n_chunks) * kVecThreads + threadIdx.x;
  const int32_t* ro = row_of + size_t(t) * top_k;
  const float* wo = topk_w + size_t(t) * top_k;
  int r[KMAX];
  float w[KMAX];
  bool any = false;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < top_k ? ro[k] : -1;
    if (r[k] >= n_rows) r[k] = -1;
    w[k] = r[k] >= 0 ? wo[k] : 0.f;
    any |= r[k] >= 0;
  }
  const bool in_self = shared_y != nullptr && t >= self_lo && t < self_hi;
  if ((!any && !in_self) || c >= row_vecs) return;
  uint4 v[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) v[k] = r[k] >= 0 ? ye[size_t(r[k]) * row_vecs + c] : make_uint4(0, 0, 0, 0);
  const uint4 vs = in_self ? shared_y[size_t(t - self_lo) * row_vecs + c] : make_uint4(0, 0, 0, 0);
  float acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (r[k] >= 0) {
      float f[EPV];
      Vec<T>::load(v[k], f);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = fmaf(w[k], f[e], acc[e]);
    }
  }
  if (in_self) {
    float f[EPV];
    Vec<T>::load(vs, f);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += f[e];
  }
  out[size_t(t) * row_vecs + c] = Vec<T>::store(acc);
}

}  // namespace
}  // namespace moe

using namespace moe;

static bool row_dtype_ok(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

static int kmax_of(int top_k) { return top_k <= 2 ? 2 : top_k <= 4 ? 4 : top_k <= 8 ? 8 : 16; }

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
  const int n_chunks = (row_vecs + kVecThreads - 1) / kVecThreads;
  if (int64_t(n_chunks) * n_tokens >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(unsigned(n_chunks * n_tokens)), block(kVecThreads);
  const uint4* xv = static_cast<const uint4*>(x);
  uint4* ov = static_cast<uint4*>(xe);
  switch (kmax_of(top_k)) {
    case 2: hipLaunchKernelGGL(dispatch_kernel<2>, grid, block, 0, stream, xv, row_vecs, n_chunks, top_k, row_of, n_rows, ov); break;
    case 4: hipLaunchKernelGGL(dispatch_kernel<4>, grid, block, 0, stream, xv, row_vecs, n_chunks, top_k, row_of, n_rows, ov); break;
    case 8: hipLaunchKernelGGL(dispatch_kernel<8>, grid, block, 0, stream, xv, row_vecs, n_chunks, top_k, row_of, n_rows, ov); break;
    default: hipLaunchKernelGGL(dispatch_kernel<16>, grid, block, 0, stream, xv, row_vecs, n_chunks, top_k, row_of, n_rows, ov); break;
  }
  return launch_status();
}

MOE_API moe_status_t moe_dispatch_blocked(const void* x, moe_dtype_t dt, int n_tokens, int hidden,
                                          const int32_t* row_token, int64_t n_rows, const int32_t* n_used, void* xe,
                                          hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (hidden % 32) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_rows == 0) return MOE_OK;
  if (!x || !row_token || !xe || !aligned16(x) || !aligned16(xe)) return MOE_ERR_INVALID_ARG;
  const int64_t units = (n_rows + 15) / 16 * ((hidden + kBlkCols - 1) / kBlkCols);
  const int64_t cap = int64_t(device_cu_count()) * 8;  // 8 workgroups per compute unit
  const dim3 grid(unsigned(units < cap ? units : cap)), block(kVecThreads);
  hipLaunchKernelGGL(dispatch_blocked_kernel, grid, block, 0, stream, static_cast<const uint4*>(x), hidden, n_tokens,
                     row_token, n_rows, n_used, static_cast<uint16_t*>(xe));
  return launch_status();
}

template <typename T, int KMAX>
static void launch_combine(dim3 grid, hipStream_t stream, const void* ye, int64_t n_rows, const int32_t* row_of,
                           const float* topk_w, int top_k, int row_vecs, int n_chunks, const void* shared_y,
                           int self_lo, int self_hi, void* out) {
  hipLaunchKernelGGL((combine_kernel<T, KMAX>), grid, dim3(kVecThreads), 0, stream, static_cast<const uint4*>(ye),
                     n_rows, row_of, topk_w, top_k, row_vecs, n_chunks, static_cast<const uint4*>(shared_y), self_lo,
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
  const int n_chunks = (row_vecs + kVecThreads - 1) / kVecThreads;
  if (int64_t(n_chunks) * n_tokens >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(unsigned(n_chunks * n_tokens));
#define MOE_COMBINE(T, KM) \
  launch_combine<T, KM>(grid, stream, ye, n_rows, row_of, topk_w, top_k, row_vecs, n_chunks, shared_y, self_lo, self_hi, out)
  const int kmax = kmax_of(top_k);
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
