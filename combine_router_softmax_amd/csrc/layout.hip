// Dispatch layout: per-(local expert, source) counts, their prefix sums, and a
// deterministic slot for every (token, k) entry.
//
// The pages give the shape of the computation (Perplexity, "Enabling
// trillion-parameter models on AWS EFA", section Dispatch and combine: count
// tokens per expert, then a prefix sum of the counts gives the offsets;
// lehuy.net, "Decoding high-performance EP kernels": the count-first layout is
// the prefix sum of the counts, the fixed-rectangle layout a static stride
// times a fixed maximum per (source rank, expert)). The kernel page counts with
// shared-memory atomics inside one block; here the order inside an expert must
// be the token order and bit-reproducible, so ranks come from wavefront
// ballots instead of atomics, and the work is spread over many workgroups:
//
//   pass 1 (hist):  one workgroup per tile of <= 64 tokens of one source;
//                   per-tile counts per local expert (LDS integer atomics:
//                   order-free, deterministic totals).
//   pass 2 (scan):  one workgroup per local expert: exclusive scan of its tile
//                   counts, per-source counts, expert totals.
//   (small layouts fold pass 2 into pass 3: each workgroup scans the tile
//   counts in LDS itself; see layout_rank_kernel)
//   pass 3 (rank):  one workgroup per tile: stable rank of each entry inside
//                   its tile (popcount over the lower lanes holding the same
//                   expert, found with one ballot per bit of the expert index,
//                   then across the 4 waves), row = tile base + rank;
//                   every workgroup also marks unused rows with -1.
//
// Tiles never straddle a source rank, so the fixed-rectangle rank inside a
// (expert, source) region is the expert's running count minus its count at
// the start of the source.
#include <mutex>

#include "moe_common.hpp"

namespace moe {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kTileTokens = 64;
constexpr int kMaxSrc = 4096;
constexpr int kMaxLocal = 1024;
constexpr int kBatch = 8;  // entries per thread whose index loads are in flight together

struct LayoutWs {
  int32_t* prefix;  // [L][tcap]: pass 1 tile counts, pass 2 turns them into exclusive prefixes
  int32_t* total;   // [L]
  int32_t* ovf;     // [L]
};

__host__ __device__ inline int tile_cap(int n_tokens, int n_src) {
  return n_src + (n_tokens + kTileTokens - 1) / kTileTokens;
}

__host__ __device__ inline LayoutWs layout_ws(void* ws, int n_local, int tcap) {
  LayoutWs w;
  int32_t* p = static_cast<int32_t*>(ws);
  w.prefix = p;
  w.total = p + size_t(n_local) * tcap;
  w.ovf = w.total + n_local;
  return w;
}

// Block-wide scan of a[0..n) in LDS: each thread folds a contiguous run, the
// run totals are scanned inside each wavefront by lane shuffles and across the
// four wavefronts through tmp, then every run is rewritten; two barriers for
// any n (a Hillis-Steele pass over 256 run totals takes sixteen). kMax:
// inclusive max-scan, returns the maximum; else exclusive sum-scan, returns
// the total. All threads must call it.
template <bool kMax>
__device__ int layout_scan(int* a, int n, int* tmp) {
  constexpr int NW = kLayoutThreads / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int id = kMax ? INT_MIN : 0;
  const int per = (n + kLayoutThreads - 1) / kLayoutThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int run = id;
  for (int i = lo; i < hi; ++i) run = kMax ? max(run, a[i]) : run + a[i];
  int incl = run;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u = __shfl_up(incl, off);
    if (lane >= off) incl = kMax ? max(incl, u) : incl + u;
  }
  if (lane == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int before = id, total = id;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    const int t = tmp[w2];
    if (w2 < w) before = kMax ? max(before, t) : before + t;
    total = kMax ? max(total, t) : total + t;
  }
  int excl = __shfl_up(incl, 1);
  if (lane == 0) excl = id;
  int carry = kMax ? max(before, excl) : before + excl;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    if (kMax) {
      carry = max(carry, v);
      a[i] = carry;
    } else {
      a[i] = carry;
      carry += v;
    }
  }
  __syncthreads();  // a[] complete, and tmp free for the next call
  return total;
}

// Source offsets repaired into [0 = off[0] <= ... <= off[S] = N], and the
// exclusive prefix ts[] of tiles per source (ts[S] = tile count). Returns the
// tile count. All threads must call it.
__device__ int build_tile_map(const int32_t* __restrict__ src_offsets, int n_src, int n_tokens, int* off, int* ts,
                              int* tmp) {
  for (int s = threadIdx.x; s <= n_src; s += kLayoutThreads) {
    int v = src_offsets[s];
    v = v < 0 ? 0 : (v > n_tokens ? n_tokens : v);
    if (s == 0) v = 0;
    if (s == n_src) v = n_tokens;
    off[s] = v;
  }
  __syncthreads();
  layout_scan<true>(off, n_src + 1, tmp);
  for (int s = threadIdx.x; s < n_src; s += kLayoutThreads)
    ts[s] = (off[s + 1] - off[s] + kTileTokens - 1) / kTileTokens;
  __syncthreads();
  const int n_tiles = layout_scan<false>(ts, n_src, tmp);
  if (threadIdx.x == 0) ts[n_src] = n_tiles;
  __syncthreads();
  return n_tiles;
}

// Source owning tile b: the last s with ts[s] <= b (empty sources are skipped).
__device__ int tile_source(const int* ts, int n_src, int b) {
  int lo = 0, hi = n_src;  // answer in [0, n_src)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ts[mid] <= b) lo = mid;
    else hi = mid;
  }
  return lo;
}

struct LayoutArgs {
  const int32_t* topk_idx;
  const int32_t* src_offsets;
  int n_tokens, top_k, n_src, expert_lo, n_local, layout, capacity, tcap;
  int64_t rows;
  LayoutWs ws;
  int32_t* counts;
  int32_t* expert_off;
  int32_t* row_of;
  int32_t* row_token;
  int32_t* status;
};

__global__ __launch_bounds__(kLayoutThreads) void layout_hist_kernel(LayoutArgs p) {
  __shared__ int off[kMaxSrc + 1];
  __shared__ int ts[kMaxSrc + 1];
  __shared__ int tmp[kLayoutThreads];
  __shared__ int hist[kMaxLocal];
  const int n_tiles = build_tile_map(p.src_offsets, p.n_src, p.n_tokens, off, ts, tmp);
  const int b = blockIdx.x;
  if (b >= n_tiles) return;
  for (int i = threadIdx.x; i < p.n_local; i += kLayoutThreads) hist[i] = 0;
  __syncthreads();
  const int s = tile_source(ts, p.n_src, b);
  const int t0 = off[s] + (b - ts[s]) * kTileTokens;
  const int t1 = min(t0 + kTileTokens, off[s + 1]);
  const int n_ent = (t1 - t0) * p.top_k;
  const int32_t* idx = p.topk_idx + size_t(t0) * p.top_k;
  // kBatch entries per thread loaded before their atomics
  for (int i0 = 0; i0 < n_ent; i0 += kBatch * kLayoutThreads) {
    unsigned le[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kLayoutThreads + threadIdx.x;
      le[u] = i < n_ent ? unsigned(idx[i]) - unsigned(p.expert_lo) : ~0u;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (le[u] < unsigned(p.n_local)) atomicAdd(&hist[le[u]], 1);
  }
  __syncthreads();
  for (int le = threadIdx.x; le < p.n_local; le += kLayoutThreads)
    p.ws.prefix[size_t(le) * p.tcap + b] = hist[le];
}

__global__ __launch_bounds__(kLayoutThreads) void layout_scan_kernel(LayoutArgs p) {
  __shared__ int off[kMaxSrc + 1];
  __shared__ int ts[kMaxSrc + 1];
  __shared__ int tmp[kLayoutThreads];
  const int n_tiles = build_tile_map(p.src_offsets, p.n_src, p.n_tokens, off, ts, tmp);
  const int le = blockIdx.x;
  int32_t* pre = p.ws.prefix + size_t(le) * p.tcap;
  const int tid = threadIdx.x;
  const int per = (n_tiles + kLayoutThreads - 1) / kLayoutThreads;
  const int lo = min(n_tiles, tid * per), hi = min(n_tiles, lo + per);
  int acc = 0;
  for (int i = lo; i < hi; ++i) acc += pre[i];
  tmp[tid] = acc;
  __syncthreads();
  for (int o = 1; o < kLayoutThreads; o <<= 1) {
    int v = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    if (tid >= o) tmp[tid] += v;
    __syncthreads();
  }
  int carry = tid ? tmp[tid - 1] : 0;
  const int total = tmp[kLayoutThreads - 1];
  for (int i = lo; i < hi; ++i) {
    const int v = pre[i];
    pre[i] = carry;
    carry += v;
  }
  __syncthreads();  // prefixes written by this block are visible to it
  int ovf = 0;
  for (int s = tid; s < p.n_src; s += kLayoutThreads) {
    const int a = ts[s] < n_tiles ? pre[ts[s]] : total;
    const int b = ts[s + 1] < n_tiles ? pre[ts[s + 1]] : total;
    const int c = b - a;
    p.counts[size_t(le) * p.n_src + s] = c;
    ovf |= c > p.capacity;
  }
  ovf = __syncthreads_or(ovf);
  if (tid == 0) {
    p.ws.total[le] = total;
    p.ws.ovf[le] = ovf;
  }
}

// FUSED (small layouts, L * (tcap + 1) <= kFusedPrefix): pass 2 is folded in.
// Every workgroup scans all experts' tile counts in LDS itself (pre[le][b] =
// the expert's count in tiles before b), and workgroup 0 writes the
// per-source counts and the status; one launch fewer.
constexpr int kFusedPrefix = 8192;

template <bool FUSED>
__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(LayoutArgs p) {
  __shared__ int off[kMaxSrc + 1];
  __shared__ int ts[kMaxSrc + 1];
  __shared__ int tmp[kLayoutThreads];
  __shared__ int start[kMaxLocal + 1];
  __shared__ int base[kMaxLocal];
  __shared__ int running[kMaxLocal];
  __shared__ int wtot[kLayoutThreads / kWave][kMaxLocal];
  extern __shared__ int pre[];  // FUSED: [L][tcap + 1]
  const int tid = threadIdx.x;
  const int L = p.n_local;
  const int n_tiles = build_tile_map(p.src_offsets, p.n_src, p.n_tokens, off, ts, tmp);
  const int PW = p.tcap + 1;  // FUSED: row pitch of pre
  if (FUSED) {
    for (int i = tid; i < L * n_tiles; i += kLayoutThreads) {
      const int le = i / n_tiles, b = i - le * n_tiles;
      pre[le * PW + b] = p.ws.prefix[size_t(le) * p.tcap + b];
    }
    __syncthreads();
    if (n_tiles >= 32) {  // uniform: a wavefront per expert, 64 tiles at a time
      const int lane = tid & (kWave - 1);
      for (int le = tid / kWave; le < L; le += kLayoutThreads / kWave) {
        int carry = 0;
        for (int b0 = 0; b0 <= n_tiles; b0 += kWave) {
          const int b = b0 + lane;
          const int v = b < n_tiles ? pre[le * PW + b] : 0;
          int incl = v;
#pragma unroll
          for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
          }
          if (b <= n_tiles) pre[le * PW + b] = carry + incl - v;  // [n_tiles]: the total
          carry += __shfl(incl, kWave - 1);
        }
      }
    } else {  // a thread per expert
      for (int le = tid; le < L; le += kLayoutThreads) {
        int acc = 0;
        for (int b = 0; b < n_tiles; ++b) {
          const int v = pre[le * PW + b];
          pre[le * PW + b] = acc;
          acc += v;
        }
        pre[le * PW + n_tiles] = acc;
      }
    }
    __syncthreads();
  }
  // (le, s) entries before tile b of expert le; the count of (le, s)
  auto prefix_at = [&](int le, int b) -> int {
    return FUSED ? pre[le * PW + b] : p.ws.prefix[size_t(le) * p.tcap + b];
  };
  auto count_of = [&](int le, int s) -> int {
    return FUSED ? pre[le * PW + ts[s + 1]] - pre[le * PW + ts[s]] : p.counts[size_t(le) * p.n_src + s];
  };

  // expert start rows (compact): exclusive scan of the totals
  for (int le = tid; le < L; le += kLayoutThreads) start[le] = FUSED ? pre[le * PW + n_tiles] : p.ws.total[le];
  __syncthreads();
  const int m_total = layout_scan<false>(start, L, tmp);
  if (tid == 0) start[L] = m_total;
  __syncthreads();
  const bool compact = p.layout == MOE_LAYOUT_COMPACT;
  const int C = p.capacity;
  const int m_kept = compact ? min(m_total, C) : 0;

  if (blockIdx.x == 0) {
    for (int le = tid; le <= L; le += kLayoutThreads)
      p.expert_off[le] = compact ? min(start[le], C) : le * p.n_src * C;
    int ovf = 0;
    if (FUSED) {
      for (int i = tid; i < L * p.n_src; i += kLayoutThreads) {
        const int le = i / p.n_src, s = i - le * p.n_src;
        const int c = count_of(le, s);
        p.counts[i] = c;
        ovf |= c > p.capacity;
      }
    } else {
      for (int le = tid; le < L; le += kLayoutThreads) ovf |= p.ws.ovf[le];
    }
    ovf = __syncthreads_or(ovf);
    if (tid == 0) p.status[0] = (compact ? (m_total > C) : (ovf != 0)) ? MOE_STATUS_OVERFLOW : 0;
  }

  // unused rows of row_token get -1 (disjoint from the rows ranked below)
  for (int64_t r = int64_t(blockIdx.x) * kLayoutThreads + tid; r < p.rows;
       r += int64_t(gridDim.x) * kLayoutThreads) {
    bool hole;
    if (compact) {
      hole = r >= m_kept;
    } else {
      const int64_t region = r / C;  // = le * S + s
      const int j = int(r - region * C);
      const int cnt = count_of(int(region / p.n_src), int(region % p.n_src));
      hole = j >= cnt;
    }
    if (hole) p.row_token[r] = -1;
  }

  const int b = blockIdx.x;
  if (b >= n_tiles) return;  // uniform per block
  const int s = tile_source(ts, p.n_src, b);
  for (int le = tid; le < L; le += kLayoutThreads) {
    const int pb = prefix_at(le, b);
    if (compact) {
      base[le] = start[le] + pb;  // row of the tile's first entry of expert le
    } else {
      const int ps = prefix_at(le, ts[s]);
      base[le] = pb - ps;  // rank inside the (le, s) region of that entry
    }
    running[le] = 0;
  }
  for (int i = tid; i < (kLayoutThreads / kWave) * L; i += kLayoutThreads) wtot[i / L][i % L] = 0;
  __syncthreads();

  const int t0 = off[s] + (b - ts[s]) * kTileTokens;
  const int t1 = min(t0 + kTileTokens, off[s + 1]);
  const int K = p.top_k;
  const int n_ent = (t1 - t0) * K;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const size_t ent0 = size_t(t0) * K;
  int nbits = 0;  // bits of a local expert index
  while ((1 << nbits) < L) ++nbits;
  int lev[kBatch];

  for (int r0 = 0; r0 < n_ent; r0 += kLayoutThreads) {
    // the indices of kBatch rounds are loaded together
    const int u = (r0 / kLayoutThreads) % kBatch;
    if (u == 0) {
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int iv = r0 + v * kLayoutThreads + tid;
        lev[v] = iv < n_ent ? int(unsigned(p.topk_idx[ent0 + iv]) - unsigned(p.expert_lo)) : -1;
      }
    }
    int le = lev[0];
#pragma unroll
    for (int v = 1; v < kBatch; ++v)
      if (u == v) le = lev[v];
    const int i = r0 + tid;
    const bool valid = i < n_ent;
    const bool local = valid && unsigned(le) < unsigned(L);
    // lanes holding the same local expert: one ballot per bit of the expert
    // index (a lane keeps the lanes that agree with it on every bit), so the
    // cost does not grow with the number of distinct experts in the wave
    uint64_t same = __ballot(local);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = local && ((le >> bit) & 1);
      const uint64_t m = __ballot(set);
      same &= set ? m : ~m;
    }
    const int in_rank = __popcll(same & lt_mask);
    if (local && in_rank == 0) wtot[w][le] = __popcll(same);  // the expert's first lane
    __syncthreads();
    if (valid) {
      int row = -1;
      if (local) {
        int rank = running[le] + in_rank;
        for (int w2 = 0; w2 < w; ++w2) rank += wtot[w2][le];
        if (compact) {
          const int rr = base[le] + rank;
          row = rr < C ? rr : -1;
        } else {
          const int j = base[le] + rank;
          row = j < C ? (le * p.n_src + s) * C + j : -1;
        }
        if (row >= 0) p.row_token[row] = t0 + i / K;
      }
      p.row_of[ent0 + i] = row;
    }
    __syncthreads();
    for (int le2 = tid; le2 < L; le2 += kLayoutThreads) {
      int add = 0;
#pragma unroll
      for (int w2 = 0; w2 < kLayoutThreads / kWave; ++w2) {
        add += wtot[w2][le2];
        wtot[w2][le2] = 0;
      }
      running[le2] += add;
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

static bool layout_desc_ok(const moe_layout_desc_t* d) {
  if (!d) return false;
  if (d->n_tokens < 0 || d->top_k < 1 || d->n_experts < 1 || d->top_k > d->n_experts) return false;
  if (d->n_src < 1 || d->n_local < 1 || d->capacity < 0) return false;
  if (d->layout != MOE_LAYOUT_COMPACT && d->layout != MOE_LAYOUT_PADDED) return false;
  return true;
}

static bool layout_desc_supported(const moe_layout_desc_t* d) {
  if (d->n_src > kMaxSrc || d->n_local > kMaxLocal) return false;
  if (int64_t(d->n_tokens) * d->top_k >= (int64_t(1) << 31)) return false;
  if (int64_t(d->n_local) * d->n_src > 65536) return false;
  return moe_layout_rows(d) < (int64_t(1) << 31);
}

MOE_API int64_t moe_layout_rows(const moe_layout_desc_t* d) {
  if (!layout_desc_ok(d)) return -1;
  if (d->layout == MOE_LAYOUT_COMPACT) return d->capacity;
  return int64_t(d->n_local) * d->n_src * d->capacity;
}

MOE_API size_t moe_dispatch_layout_workspace(const moe_layout_desc_t* d) {
  if (!layout_desc_ok(d)) return 0;
  const size_t tcap = size_t(tile_cap(d->n_tokens, d->n_src));
  return align_up((size_t(d->n_local) * tcap + 2 * size_t(d->n_local)) * sizeof(int32_t), 256);
}

// Scratch of the allocation-free entry point: the layout's tile-count
// workspace in a file-scope device array, one copy per GPU, kept until the
// process ends. The host never passes the array's name to a kernel (in host
// code it only stands for the symbol): its device address is looked up once
// per device with hipGetSymbolAddress and cached.
constexpr size_t kLayoutScratchBytes = size_t(4) << 20;
__device__ __align__(256) char layout_scratch[kLayoutScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kScratchMaxDevices] = {};

// Device address of the current device's scratch array (nullptr on failure).
void* layout_scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(layout_scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}
}  // namespace

MOE_API moe_status_t moe_dispatch_layout_noalloc(const moe_layout_desc_t* d, const int32_t* topk_idx,
                                                 const int32_t* src_offsets, int32_t* counts, int32_t* expert_off,
                                                 int32_t* row_of, int32_t* row_token, int32_t* status,
                                                 hipStream_t stream) {
  if (!layout_desc_ok(d)) return MOE_ERR_INVALID_ARG;
  if (!layout_desc_supported(d)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe_dispatch_layout_workspace(d);
  if (need > kLayoutScratchBytes) return MOE_ERR_UNSUPPORTED;  // beyond the fixed scratch
  void* ws = layout_scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  // every word of the scratch a call reads is written earlier in the same
  // call (tile counts, then their prefixes), so nothing needs clearing
  return moe_dispatch_layout(d, topk_idx, src_offsets, counts, expert_off, row_of, row_token, status, ws, need,
                             stream);
}

MOE_API moe_status_t moe_dispatch_layout(const moe_layout_desc_t* d, const int32_t* topk_idx,
                                         const int32_t* src_offsets, int32_t* counts, int32_t* expert_off,
                                         int32_t* row_of, int32_t* row_token, int32_t* status, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  if (!layout_desc_ok(d)) return MOE_ERR_INVALID_ARG;
  if (!layout_desc_supported(d)) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = moe_layout_rows(d);
  if (!src_offsets || !counts || !expert_off || !status) return MOE_ERR_INVALID_ARG;
  if (d->n_tokens > 0 && (!topk_idx || !row_of)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && !row_token) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < moe_dispatch_layout_workspace(d)) return MOE_ERR_WORKSPACE;

  LayoutArgs p;
  p.topk_idx = topk_idx;
  p.src_offsets = src_offsets;
  p.n_tokens = d->n_tokens;
  p.top_k = d->top_k;
  p.n_src = d->n_src;
  p.expert_lo = d->expert_lo;
  p.n_local = d->n_local;
  p.layout = d->layout;
  p.capacity = d->capacity;
  p.tcap = tile_cap(d->n_tokens, d->n_src);
  p.rows = rows;
  p.ws = layout_ws(ws, d->n_local, p.tcap);
  p.counts = counts;
  p.expert_off = expert_off;
  p.row_of = row_of;
  p.row_token = row_token;
  p.status = status;

  const dim3 block(kLayoutThreads);
  hipLaunchKernelGGL(layout_hist_kernel, dim3(p.tcap), block, 0, stream, p);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const int64_t pre_ints = int64_t(d->n_local) * (p.tcap + 1);
  if (pre_ints <= kFusedPrefix) {
    hipLaunchKernelGGL(layout_rank_kernel<true>, dim3(p.tcap), block, size_t(pre_ints) * sizeof(int), stream, p);
    return launch_status();
  }
  hipLaunchKernelGGL(layout_scan_kernel, dim3(d->n_local), block, 0, stream, p);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  hipLaunchKernelGGL(layout_rank_kernel<false>, dim3(p.tcap), block, 0, stream, p);
  return launch_status();
}
