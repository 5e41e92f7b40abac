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

// Workgroup b handles PPT * 256 consecutive 16-byte pieces of token
// t = b / n_chunks (thread i: pieces i, i + 256, ...): the token's slots are
// uniform per workgroup (scalar loads); every thread has PPT loads in flight
// and stores each piece to each slot.
// BLOCKED: xe in the 16-row blocked layout (blocks of 16 rows x 32 columns,
// 1 KiB each): piece c of row r (8 columns) goes to block (r / 16, c / 4),
// row r % 16, 16-byte slot c % 4; four neighbouring lanes still write 64
// contiguous bytes.
constexpr int kDispatchPpt = 4;
template <int KMAX, bool BLOCKED>
__global__ __launch_bounds__(kVecThreads) void dispatch_kernel(const uint4* __restrict__ x, int row_vecs, int n_chunks,
                                                                int n_tokens, int top_k,
                                                                const int32_t* __restrict__ row_of, int64_t n_rows,
                                                                uint4* __restrict__ xe) {
  (void)n_tokens;
  const int t = blockIdx.x / n_chunks;
  const int c0 = (blockIdx.x - t * n_chunks) * kVecThreads * kDispatchPpt + threadIdx.x;
  const int32_t* ro = row_of + size_t(t) * top_k;
  int r[KMAX];
  bool any = false;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < top_k ? ro[k] : -1;
    if (r[k] >= n_rows) r[k] = -1;
    any |= r[k] >= 0;
  }
  if (!any || c0 >= row_vecs) return;
  uint4 v[kDispatchPpt];
#pragma unroll
  for (int i = 0; i < kDispatchPpt; ++i)  // unconditional loads (a tail piece repeats a valid one)
    v[i] = x[size_t(t) * row_vecs + min(c0 + i * kVecThreads, row_vecs - 1)];
  // keep the pieces in registers: without this the compiler reloads each one
  // from memory before every slot's store
#pragma unroll
  for (int i = 0; i < kDispatchPpt; ++i) asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (r[k] >= 0) {
#pragma unroll
      for (int i = 0; i < kDispatchPpt; ++i) {
        const int c = c0 + i * kVecThreads;
        if (c >= row_vecs) continue;
        if (BLOCKED) {
          const size_t blk = size_t(r[k] >> 4) * size_t(row_vecs >> 2) + size_t(c >> 2);
          xe[blk * 64 + size_t(r[k] & 15) * 4 + (c & 3)] = v[i];
        } else {
          xe[size_t(r[k]) * row_vecs + c] = v[i];
        }
      }
    }
}

// The scales of fp8 payload rows: xes[row_of[t*K+k]][j] = xs[t][j] (one
// workgroup of one wave per token; a row holds hidden / 128 scales).
__global__ __launch_bounds__(kWave) void dispatch_scales_kernel(const float* __restrict__ xs, int per_row,
                                                                int top_k, const int32_t* __restrict__ row_of,
                                                                int64_t n_rows, float* __restrict__ xes) {
  const int t = blockIdx.x;
  for (int k = 0; k < top_k; ++k) {
    const int r = row_of[size_t(t) * top_k + k];
    if (r < 0 || r >= n_rows) continue;  // uniform
    for (int j = threadIdx.x; j < per_row; j += kWave) xes[size_t(r) * per_row + j] = xs[size_t(t) * per_row + j];
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

// Same decomposition as dispatch: workgroup b handles PPT * 256 16-byte pieces
// of token t = b / n_chunks. The token's kept entries (uniform per workgroup:
// scalar) are taken in ascending k, KG at a time: the pieces of those KG rows
// (and, with the first group, of the shared-expert row) are all in flight
// together, then accumulated in k order; a token with at most KG rows on this
// GPU - the usual case - costs one round trip. The registers held are PPT x KG
// pieces, not PPT x K.
// MULTI: leave tokens with exactly one kept entry outside [self_lo, self_hi)
// (the down projection's scatter wrote them).
template <typename T, int KMAX, int PPT, int KG, bool MULTI>
__device__ __forceinline__ void combine_token(const uint4* __restrict__ ye, int64_t n_rows,
                                              const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
                                              int top_k, int row_vecs, const uint4* __restrict__ shared_y,
                                              int self_lo, int self_hi, uint4* __restrict__ out, int t, int chunk) {
  constexpr int EPV = Vec<T>::N;
  const int c0 = chunk * kVecThreads * PPT + threadIdx.x;
  const int32_t* ro = row_of + size_t(t) * top_k;
  const float* wo = topk_w + size_t(t) * top_k;
  int r[KMAX];
  float w[KMAX];
  uint32_t kept = 0;  // bit k: entry k is a row of this GPU
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < top_k ? ro[k] : -1;
    if (r[k] >= n_rows) r[k] = -1;
    w[k] = r[k] >= 0 ? wo[k] : 0.f;
    kept |= r[k] >= 0 ? 1u << k : 0u;
  }
  const bool in_self = shared_y != nullptr && t >= self_lo && t < self_hi;
  if ((kept == 0 && !in_self) || c0 >= row_vecs) return;
  if (MULTI && __builtin_popcount(kept) == 1 && !(t >= self_lo && t < self_hi)) return;
  int cs[PPT];  // piece indices (a tail piece repeats a valid one; its result is not stored)
#pragma unroll
  for (int i = 0; i < PPT; ++i) cs[i] = min(c0 + i * kVecThreads, row_vecs - 1);
  uint4 vs[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    vs[i] = in_self ? shared_y[size_t(t - self_lo) * row_vecs + cs[i]] : make_uint4(0, 0, 0, 0);
  float acc[PPT][EPV];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[i][e] = 0.f;
  // entry k's rank among the kept ones (scalar); round j takes ranks
  // j KG .. j KG + KG - 1. (Slots are chosen by comparing ranks, every array
  // index static: a select on a computed index would be turned back into an
  // indexed array, which the compiler keeps in memory.)
  int rank[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) rank[k] = (kept >> k & 1u) ? __builtin_popcount(kept & ((1u << k) - 1u)) : -1;
  const int n_kept = __builtin_popcount(kept);
  for (int j0 = 0; j0 < n_kept; j0 += KG) {  // uniform
    int rg[KG];
    float wg[KG];
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      if constexpr (KG >= KMAX) {  // one round: every entry in its own slot
        rg[g] = r[g];
        wg[g] = w[g];
      } else {
        rg[g] = -1;
        wg[g] = 0.f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const bool hit = rank[k] == j0 + g;
          rg[g] = hit ? r[k] : rg[g];
          wg[g] = hit ? w[k] : wg[g];
        }
      }
    }
    uint4 v[PPT][KG];
#pragma unroll
    for (int i = 0; i < PPT; ++i)
#pragma unroll
      for (int g = 0; g < KG; ++g)
        v[i][g] = rg[g] >= 0 ? ye[size_t(rg[g]) * row_vecs + cs[i]] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PPT; ++i)
#pragma unroll
      for (int g = 0; g < KG; ++g)
        if (rg[g] >= 0) {
          float f[EPV];
          Vec<T>::load(v[i][g], f);
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[i][e] = fmaf(wg[g], f[e], acc[i][e]);
        }
  }
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int c = c0 + i * kVecThreads;
    if (in_self) {
      float f[EPV];
      Vec<T>::load(vs[i], f);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[i][e] += f[e];
    }
    if (c < row_vecs) out[size_t(t) * row_vecs + c] = Vec<T>::store(acc[i]);
  }
}

template <typename T, int KMAX, int PPT, int KG, bool MULTI>
__global__ __launch_bounds__(kVecThreads) void combine_kernel(
    const uint4* __restrict__ ye, int64_t n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
    int top_k, int row_vecs, int n_chunks, const uint4* __restrict__ shared_y, int self_lo, int self_hi,
    uint4* __restrict__ out) {
  const int t = blockIdx.x / n_chunks;
  combine_token<T, KMAX, PPT, KG, MULTI>(ye, n_rows, row_of, topk_w, top_k, row_vecs, shared_y, self_lo, self_hi,
                                         out, t, blockIdx.x - t * n_chunks);
}

// Few local experts (rows on this GPU well below tokens x K): most tokens have
// nothing here, and a workgroup per token spends the launch on workgroups that
// read K indices and leave. Instead workgroup w takes the kSparseTokens tokens
// w, w + G, w + 2G, ... (strided, so the self range, where every token has a
// row, spreads over the grid): one thread per (token, entry) tests the entry,
// the tokens with a kept entry or a shared row are marked in one LDS word,
// and the workgroup combines just those, in token order, as above. The
// workgroup with the most touched tokens sets the time (one round trip per
// token), so the batches are small: 4 tokens, not 2, 8 or 16 (measured at the
// EP128 decode share: 14.8, 14.1, 16.9, 21.1 us per call against 18.6 for a
// workgroup per token).
constexpr int kSparseTokens = 4;

template <typename T, int KMAX, int PPT, int KG, bool MULTI>
__global__ __launch_bounds__(kVecThreads) void combine_sparse_kernel(
    const uint4* __restrict__ ye, int64_t n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w,
    int n_tokens, int top_k, int row_vecs, int n_chunks, const uint4* __restrict__ shared_y, int self_lo, int self_hi,
    uint4* __restrict__ out) {
  static_assert(kSparseTokens * KMAX <= kVecThreads, "one thread per (token, entry)");
  __shared__ uint32_t touched;
  const int G = gridDim.x;
  if (threadIdx.x == 0) touched = 0u;
  __syncthreads();
  if (threadIdx.x < kSparseTokens * KMAX) {
    const int j = threadIdx.x / KMAX, k = threadIdx.x % KMAX;
    const int t = int(blockIdx.x) + j * G;
    if (t < n_tokens) {
      const int r = k < top_k ? row_of[size_t(t) * top_k + k] : -1;
      const bool self = shared_y != nullptr && k == 0 && t >= self_lo && t < self_hi;
      if ((r >= 0 && r < n_rows) || self) atomicOr(&touched, 1u << j);
    }
  }
  __syncthreads();
  uint32_t m = __builtin_amdgcn_readfirstlane(touched);
  while (m) {  // uniform
    const int j = __builtin_ctz(m);
    m &= m - 1u;
    const int t = int(blockIdx.x) + j * G;
    for (int c = 0; c < n_chunks; ++c)
      combine_token<T, KMAX, PPT, KG, MULTI>(ye, n_rows, row_of, topk_w, top_k, row_vecs, shared_y, self_lo, self_hi,
                                             out, t, c);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

static bool row_dtype_ok(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

static int kmax_of(int top_k) { return top_k <= 2 ? 2 : top_k <= 4 ? 4 : top_k <= 8 ? 8 : 16; }

// One workgroup per (token, chunk) unit.
static unsigned vec_grid(int64_t units) { return unsigned(units > 0 ? units : 1); }

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
  const int n_chunks = (row_vecs + kVecThreads * kDispatchPpt - 1) / (kVecThreads * kDispatchPpt);
  if (int64_t(n_chunks) * n_tokens >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(vec_grid(int64_t(n_chunks) * n_tokens)), block(kVecThreads);
  const uint4* xv = static_cast<const uint4*>(x);
  uint4* ov = static_cast<uint4*>(xe);
  switch (kmax_of(top_k)) {
    case 2: hipLaunchKernelGGL((dispatch_kernel<2, false>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    case 4: hipLaunchKernelGGL((dispatch_kernel<4, false>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    case 8: hipLaunchKernelGGL((dispatch_kernel<8, false>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    default: hipLaunchKernelGGL((dispatch_kernel<16, false>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
  }
  return launch_status();
}

MOE_API moe_status_t moe_dispatch_fp8(const uint8_t* xq, const float* xs, int n_tokens, int hidden, int top_k,
                                      const int32_t* row_of, int64_t n_rows, uint8_t* xeq, float* xes,
                                      hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || top_k < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (hidden % 128) return MOE_ERR_UNSUPPORTED;
  if (top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (n_tokens == 0 || n_rows == 0) return MOE_OK;
  if (!xs || !xes || (reinterpret_cast<uintptr_t>(xs) & 3u) || (reinterpret_cast<uintptr_t>(xes) & 3u))
    return MOE_ERR_INVALID_ARG;
  // the codes are rows of hidden bytes: the bf16/f32 row copy moves them bit for bit
  const moe_status_t st = moe_dispatch(xq, MOE_BF16, n_tokens, hidden / 2, top_k, row_of, n_rows, xeq, stream);
  if (st != MOE_OK) return st;
  hipLaunchKernelGGL(dispatch_scales_kernel, dim3(unsigned(n_tokens)), dim3(kWave), 0, stream, xs, hidden / 128,
                     top_k, row_of, n_rows, xes);
  return launch_status();
}

MOE_API moe_status_t moe_dispatch_blocked(const void* x, moe_dtype_t dt, int n_tokens, int hidden, int top_k,
                                          const int32_t* row_of, int64_t n_rows, void* xe, hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || top_k < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (hidden % 32) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_rows == 0) return MOE_OK;
  if (!x || !row_of || !xe || !aligned16(x) || !aligned16(xe)) return MOE_ERR_INVALID_ARG;
  const int row_vecs = hidden / 8;
  const int n_chunks = (row_vecs + kVecThreads * kDispatchPpt - 1) / (kVecThreads * kDispatchPpt);
  if (int64_t(n_chunks) * n_tokens >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  const dim3 grid(vec_grid(int64_t(n_chunks) * n_tokens)), block(kVecThreads);
  const uint4* xv = static_cast<const uint4*>(x);
  uint4* ov = static_cast<uint4*>(xe);
  switch (kmax_of(top_k)) {
    case 2: hipLaunchKernelGGL((dispatch_kernel<2, true>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    case 4: hipLaunchKernelGGL((dispatch_kernel<4, true>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    case 8: hipLaunchKernelGGL((dispatch_kernel<8, true>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
    default: hipLaunchKernelGGL((dispatch_kernel<16, true>), grid, block, 0, stream, xv, row_vecs, n_chunks, n_tokens, top_k, row_of, n_rows, ov); break;
  }
  return launch_status();
}

// Two shapes. From about a thousand tokens: 4 pieces per thread (a 7168-wide
// bf16 row is one workgroup) and 2 kept rows per round trip, the most bytes
// in flight per register (measured best from 1024 tokens of a 7168-wide
// layer up). Smaller batches: 2 pieces per thread (twice the workgroups) and
// all K rows in one round trip, so no token costs more than one.
constexpr int kCombineManyTokens = 1024;

template <typename T, int KMAX, int PPT, int KG, bool MULTI>
static void launch_combine(hipStream_t stream, const void* ye, int64_t n_rows, const int32_t* row_of,
                           const float* topk_w, int n_tokens, int top_k, int row_vecs, const void* shared_y,
                           int self_lo, int self_hi, void* out) {
  const int n_chunks = (row_vecs + kVecThreads * PPT - 1) / (kVecThreads * PPT);
  // rows for at most half the (token, entry) pairs: at most half the experts
  // a token picks can be local, and few tokens are touched
  if (int64_t(n_rows) * 2 <= int64_t(n_tokens) * top_k) {
    const dim3 grid(unsigned((n_tokens + kSparseTokens - 1) / kSparseTokens));
    hipLaunchKernelGGL((combine_sparse_kernel<T, KMAX, PPT, KG, MULTI>), grid, dim3(kVecThreads), 0, stream,
                       static_cast<const uint4*>(ye), n_rows, row_of, topk_w, n_tokens, top_k, row_vecs, n_chunks,
                       static_cast<const uint4*>(shared_y), self_lo, self_hi, static_cast<uint4*>(out));
    return;
  }
  const dim3 grid(vec_grid(int64_t(n_chunks) * n_tokens));
  hipLaunchKernelGGL((combine_kernel<T, KMAX, PPT, KG, MULTI>), grid, dim3(kVecThreads), 0, stream,
                     static_cast<const uint4*>(ye), n_rows, row_of, topk_w, top_k, row_vecs, n_chunks,
                     static_cast<const uint4*>(shared_y), self_lo, self_hi, static_cast<uint4*>(out));
}

template <typename T, int KMAX, bool MULTI>
static void launch_combine(hipStream_t stream, const void* ye, int64_t n_rows, const int32_t* row_of,
                           const float* topk_w, int n_tokens, int top_k, int row_vecs, const void* shared_y,
                           int self_lo, int self_hi, void* out) {
  if (n_tokens >= kCombineManyTokens)
    launch_combine<T, KMAX, 4, 2, MULTI>(stream, ye, n_rows, row_of, topk_w, n_tokens, top_k, row_vecs, shared_y,
                                         self_lo, self_hi, out);
  else
    launch_combine<T, KMAX, 2, KMAX, MULTI>(stream, ye, n_rows, row_of, topk_w, n_tokens, top_k, row_vecs, shared_y,
                                            self_lo, self_hi, out);
}

template <bool MULTI>
static moe_status_t combine_entry(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                                  const float* topk_w, int n_tokens, int top_k, int hidden, const void* shared_y,
                                  int self_lo, int self_hi, void* out, hipStream_t stream) {
  if (n_tokens < 0 || hidden < 1 || top_k < 1 || n_rows < 0) return MOE_ERR_INVALID_ARG;
  if (!row_dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (top_k > kMaxK) return MOE_ERR_UNSUPPORTED;
  const size_t row_bytes = size_t(hidden) * dtype_size(dt);
  if (row_bytes % 16) return MOE_ERR_INVALID_ARG;
  if ((shared_y || MULTI) && (self_lo < 0 || self_hi < self_lo || self_hi > n_tokens)) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  if (!row_of || !topk_w || !out || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  if (n_rows > 0 && (!ye || !aligned16(ye))) return MOE_ERR_INVALID_ARG;
  if (shared_y && !aligned16(shared_y)) return MOE_ERR_INVALID_ARG;
  const int row_vecs = int(row_bytes / 16);
  const int n_chunks = (row_vecs + kVecThreads * 2 - 1) / (kVecThreads * 2);  // the smaller pieces' count
  if (int64_t(n_chunks) * n_tokens >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
#define MOE_COMBINE(T, KM) \
  launch_combine<T, KM, MULTI>(stream, ye, n_rows, row_of, topk_w, n_tokens, top_k, row_vecs, shared_y, self_lo, \
                               self_hi, out)
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

MOE_API moe_status_t moe_combine(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                                 const float* topk_w, int n_tokens, int top_k, int hidden, const void* shared_y,
                                 int self_lo, int self_hi, void* out, hipStream_t stream) {
  return combine_entry<false>(ye, dt, n_rows, row_of, topk_w, n_tokens, top_k, hidden, shared_y, self_lo, self_hi,
                              out, stream);
}

MOE_API moe_status_t moe_combine_multi(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                                       const float* topk_w, int n_tokens, int top_k, int hidden,
                                       const void* shared_y, int self_lo, int self_hi, void* out,
                                       hipStream_t stream) {
  return combine_entry<true>(ye, dt, n_rows, row_of, topk_w, n_tokens, top_k, hidden, shared_y, self_lo, self_hi,
                             out, stream);
}
