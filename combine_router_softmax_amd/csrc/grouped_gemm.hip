// Grouped SwiGLU expert FFN (Perplexity, "Lower latency and higher throughput
// with multi-node DeepSeek deployment", sections GroupGEMM and Quantization).
//
// Two products per expert g over the rows it holds:
//   up   : h = silu(A W_gate^T) * (A W_up^T)   A [m_g, H], W13 [2I, H]  -> h [m_g, I]
//   down : y = h W2^T                          W2 [H, I]               -> y [m_g, H]
// Both are "NT" products: activations and weights are contiguous along the
// reduction dimension.
//
// Work decomposition (routing-aware, persistent; the page's point that kernels
// must read the per-expert counts on the device rather than size the work from
// the buffer bound): a fixed grid of workgroups walks a tile list built in
// every workgroup from the device counts. A tile is (expert, 128-row block,
// N block); row blocks are the fastest index, so workgroups that share a
// weight block run side by side and the weight block is fetched from HBM
// once. Empty experts produce no tiles.
//
// Decode tile (4 waves, ffn_bf16_kernel): up = 64 rows x 64 h columns, i.e.
// 64 gate + 64 up weight rows; down = 64 rows x 128 output columns. Each wave
// owns 32 weight rows (up: 16 gate + the 16 matching up rows, so SwiGLU pairs
// land in one lane) and all row blocks. MFMA v_mfma_f32_32x32x16_bf16 with the
// weights as the A operand (32 weight rows) and the activations as the B
// operand (32 rows); 32-row blocks with no rows are skipped, so a decode
// expert with ~32 rows costs one MFMA column block while the weights stream
// once.
//
// Data path per 128-deep K chunk: each lane loads its weight row's pieces
// straight from HBM into registers (chunks ahead), and the workgroup stages
// the activation chunk [64 rows x 128] in LDS by LDS DMA (one barrier per
// chunk). The reduction order inside a chunk is permuted identically for both
// operands so every weight load is a 64-byte run. Groups with many rows take
// the wide-tile kernel instead.
//
// fp8 e4m3 weights (ffn_fp8_kernel): each code is decoded exactly to fp32,
// multiplied by its 128x128 block's fp32 scale and rounded once to bf16 in
// registers, then the bf16 MFMA runs as for bf16 weights (W8A16).
//
// fp32 activations + fp32 weights (small parity problems) use a plain SIMT
// kernel with the same scheduler.
#include <algorithm>
#include <type_traits>

#include "moe_common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kMaxGemmThreads = 512;  // the fp8 decode kernel's workgroup
constexpr int kBM = 128;            // rows per tile
constexpr int kMB = kBM / 32;       // 32-row MFMA blocks per tile
constexpr int kKC = 128;            // reduction chunk
constexpr int kMaxGroups = 512;
constexpr int kGemmMaxSrc = 512;

enum { kUp = 0, kDown = 1 };

// wide-tile kernel (groups with many rows)
constexpr int kWN = 256;             // weight rows per wide tile
constexpr int kWM = 256;             // activation rows per wide tile
constexpr int kWK = 32;              // reduction depth per LDS stage (32 or 64)
constexpr int kWideGrid = 256;       // one workgroup per compute unit
constexpr int kWideMinRows = 128;    // a group with at least this many rows may take the wide kernel ...
constexpr int kWideMinTiles = 16;    // ... if the launch then has at least this many wide tiles
constexpr int kNoWide = 0x7fffffff;  // wide_min when the wide kernel is not used

struct GemmArgs {
  // routed experts
  const void* a;              // [rows, K] activations (x for up, h for down)
  int64_t rows;               // R
  const int32_t* counts;      // [G, S] (padded)
  const int32_t* group_off;   // [G + 1] (compact)
  int G, S, C, layout;
  const void* w;              // [G, n_w_rows, K]
  const float* s;             // fp8: [G, n_w_rows/128, K/128]
  void* out;                  // [rows, n_out]
  // optional shared expert: one more group (index G) over rows [0, sh_rows) of its own buffers
  const void* sh_a;
  const void* sh_w;
  const float* sh_s;
  void* sh_out;
  int sh_rows;                // 0 = none
  int n_w_rows;               // 2I (up) or H (down)
  int K;                      // reduction length
  int n_out;                  // I (up) or H (down)
  int n_tiles_n;              // N tiles per expert (decode-shaped kernels)
  int packed;                 // weights in the packed (load-order) layout
  int wide_min;               // groups with at least this many rows may go to the wide-tile kernel ...
  int wide_min_tiles;         // ... if the wide groups make at least this many wide tiles
  int a_blk, sh_a_blk;        // routed / shared activations in the 16-row blocked layout
  int out_blk;                // outputs (routed and shared) in the 16-row blocked layout
  const int32_t* a_rows;      // routed input row r is row a_rows[r] of a (nullptr: row r)
  int a_nrows;                // rows of a when gathering
};

// 16-row blocked activation layout: element (r, c) of an [R, K] matrix sits
// at ((r / 16) * (K / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32, i.e.
// blocks of 16 rows x 32 columns (1 KiB of bf16) stored contiguously, the
// blocks of one 16-row group in column order. A wave load of 16 rows x 32
// columns is then one contiguous KiB instead of 16 separate 64-byte pieces.
__device__ __forceinline__ size_t blk_row_base(int64_t r, int K) {
  return size_t(r >> 4) * size_t(K >> 5) * 512 + size_t(r & 15) * 32;
}
__device__ __forceinline__ size_t act_off(int64_t r, int c, int K, bool blk) {
  return blk ? blk_row_base(r, K) + size_t(c >> 5) * 512 + (c & 31) : size_t(r) * K + c;
}

constexpr int kGatherRows = 256;  // tile rows of the kernels that gather (bf16 64, fp8 96, wide 256)

struct Sched {
  int tile_start[kMaxGroups + 2];
  int m[kMaxGroups + 1];
  int seg[kGemmMaxSrc + 1];
  union {
    int rowmap[256];
    int tmp[kMaxGemmThreads];  // scan scratch: every scan ends before a rowmap is written
  };
  int arow[kGatherRows];       // gathering: the input row of each tile row
  int cur_seg_group;
  int wide_tiles;
};

// Rows per group from the device counts (clamped so every row stays inside
// [0, rows)), then the exclusive prefix of tiles per group. Schedule order:
// the shared expert first (its rows are always present, so its tiles start
// with the first wave of workgroups instead of forming a tail), then the
// routed experts. Only groups on the kernel's side get tiles: the launch goes
// wide if the groups with m >= wide_min make at least wide_min_tiles wide
// tiles, and then every group is wide; otherwise the stream-K kernel takes
// them all. Both kernels evaluate this identically from the same counts.
// Returns the tile count. All threads must call it.
template <int NT = kGemmThreads>
__device__ __forceinline__ int build_schedule(const GemmArgs& p, int bm, int ntn, bool wide, Sched& sh) {
  const int tid = threadIdx.x;
  const int nsh = p.sh_rows > 0 ? 1 : 0;
  const int Gt = p.G + nsh;
  if (p.layout == MOE_LAYOUT_COMPACT) {
    for (int g = tid; g < p.G; g += NT) {
      const int64_t lo = min<int64_t>(max<int64_t>(p.group_off[g], 0), p.rows);
      const int64_t hi = min<int64_t>(max<int64_t>(p.group_off[g + 1], lo), p.rows);
      sh.m[nsh + g] = int(hi - lo);
    }
  } else {
    for (int g = tid; g < p.G; g += NT) sh.m[nsh + g] = 0;
    __syncthreads();
    for (int i = tid; i < p.G * p.S; i += NT) {
      const int c = min(max(p.counts[i], 0), p.C);
      if (c) atomicAdd(&sh.m[nsh + i / p.S], c);
    }
  }
  if (tid == 0) {
    if (nsh) sh.m[0] = p.sh_rows;
    sh.wide_tiles = 0;
  }
  __syncthreads();
  if (p.wide_min != kNoWide) {
    int wt = 0;
    for (int g = tid; g < Gt; g += NT)
      if (sh.m[g] >= p.wide_min) wt += (sh.m[g] + kWM - 1) / kWM * (p.n_w_rows / kWN);
    if (wt) atomicAdd(&sh.wide_tiles, wt);
    __syncthreads();
  }
  // once the launch qualifies, every group takes the wide kernel (one launch
  // does all the work; small groups are cheap ragged tiles there)
  const int wide_min = sh.wide_tiles >= p.wide_min_tiles ? 1 : kNoWide;
  for (int g = tid; g < Gt; g += NT) {
    const int m = sh.m[g];
    sh.tile_start[g] = ((m >= wide_min) == wide) ? (m + bm - 1) / bm * ntn : 0;
  }
  __syncthreads();
  const int total = block_scan_lds<false, NT>(sh.tile_start, Gt, sh.tmp);
  if (tid == 0) {
    sh.tile_start[Gt] = total;
    sh.cur_seg_group = -1;
  }
  __syncthreads();
  // uniform (every thread read the same LDS word): scalar registers, so the
  // work split derived from it stays scalar
  return __builtin_amdgcn_readfirstlane(total);
}

// c ? a : b on values: the operands are read before the choice. (On the two
// fields themselves the conditional is an lvalue, which the compiler may
// lower to a load from a chosen field address; that keeps the whole kernel
// argument block in scratch memory.)
template <class T>
__device__ __forceinline__ T pick(bool c, T a, T b) {
  return c ? a : b;
}

struct Tile {
  int g;        // routed expert index (unused for the shared expert)
  int we;       // expert index inside the weight tensor of the tile's problem
  bool shared;
  int nt, r0, nrows;
  int mtiles;   // row tiles of the tile's group (1: its weights are read once)
};

// Tile order inside a group. Default: row tiles fastest (consecutive tiles
// share a weight block). BLOCKED: the N tiles are cut into blocks of nbw (4
// when they divide evenly), and inside a block the order is (row tile, N
// tile); so any 32 consecutive tiles cover a compact rectangle of row tiles x
// N tiles (8 x 4 when the group has 8 row tiles), i.e. 12 distinct operand
// slabs instead of 2 + 16 (N fastest) or 32 + 1 (rows fastest).
template <bool BLOCKED = false>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, int bm, int ntn, const Sched& sh, int t) {
  const int nsh = p.sh_rows > 0 ? 1 : 0;
  const int Gt = p.G + nsh;
  int lo = 0, hi = Gt;  // last q with tile_start[q] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sh.tile_start[mid] <= t) lo = mid;
    else hi = mid;
  }
  Tile tl;
  tl.shared = lo < nsh;
  tl.g = tl.shared ? 0 : lo - nsh;
  tl.we = tl.g;
  const int local = t - sh.tile_start[lo];
  const int mtiles = (sh.m[lo] + bm - 1) / bm;
  tl.mtiles = mtiles;
  if (BLOCKED) {
    const int nbw = ntn % 4 == 0 ? 4 : (ntn % 2 == 0 ? 2 : 1);
    const int blk = local / (nbw * mtiles), rem = local % (nbw * mtiles);
    tl.nt = blk * nbw + rem % nbw;
    tl.r0 = (rem / nbw) * bm;
  } else {
    tl.nt = local / mtiles;
    tl.r0 = (local % mtiles) * bm;
  }
  tl.nrows = min(bm, sh.m[lo] - tl.r0);
  // every caller passes a workgroup-uniform t, so the fields are uniform; the
  // compiler cannot see that through the LDS reads: scalar registers (loop
  // bounds and weight addresses derived from them then stay scalar)
  tl.g = __builtin_amdgcn_readfirstlane(tl.g);
  tl.we = __builtin_amdgcn_readfirstlane(tl.we);
  tl.shared = __builtin_amdgcn_readfirstlane(int(tl.shared)) != 0;
  tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
  tl.r0 = __builtin_amdgcn_readfirstlane(tl.r0);
  tl.nrows = __builtin_amdgcn_readfirstlane(tl.nrows);
  tl.mtiles = __builtin_amdgcn_readfirstlane(tl.mtiles);
  return tl;
}

// Physical row of each of the tile's rows (-1 past the group's rows).
template <int NT = kGemmThreads>
__device__ __forceinline__ void build_rowmap(const GemmArgs& p, const Tile& tl, int bm, Sched& sh,
                                             bool input_rows = false) {
  const int tid = threadIdx.x;
  // gathering (kernels that read their input through sh.arow): the input row
  // of each present row, clamped into a's rows
  const bool gat = input_rows && p.a_rows != nullptr && !tl.shared && bm <= kGatherRows;
  auto put = [&](int phys) {
    sh.rowmap[tid] = phys;
    if (gat) sh.arow[tid] = phys >= 0 ? min(max(p.a_rows[phys], 0), p.a_nrows - 1) : -1;
  };
  if (tl.shared || p.layout == MOE_LAYOUT_COMPACT) {
    if (tid < bm) {
      const int64_t base = tl.shared ? 0 : min<int64_t>(max<int64_t>(p.group_off[tl.g], 0), p.rows);
      put(tid < tl.nrows ? int(base + tl.r0 + tid) : -1);
    }
    __syncthreads();
    return;
  }
  if (sh.cur_seg_group != tl.g) {  // uniform: every thread reads the same LDS word
    __syncthreads();
    for (int s = tid; s < p.S; s += NT) sh.seg[s] = min(max(p.counts[tl.g * p.S + s], 0), p.C);
    __syncthreads();
    const int tot = block_scan_lds<false, NT>(sh.seg, p.S, sh.tmp);
    if (tid == 0) {
      sh.seg[p.S] = tot;
      sh.cur_seg_group = tl.g;
    }
    __syncthreads();
  }
  if (tid < bm) {
    int phys = -1;
    if (tid < tl.nrows) {
      const int li = tl.r0 + tid;
      int lo = 0, hi = p.S;  // last s with seg[s] <= li
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sh.seg[mid] <= li) lo = mid;
        else hi = mid;
      }
      phys = (tl.g * p.S + lo) * p.C + (li - sh.seg[lo]);
    }
    put(phys);
  }
  __syncthreads();
}

// A pointer every lane of the wave holds, moved into scalar registers (values
// read from LDS are not known to be uniform): loads can then take it as their
// scalar base with a 32-bit per-lane offset, so no per-lane 64-bit address
// register is computed (and freed) per load.
// (The result is a global-address-space pointer: rebuilt from integers, a
// generic pointer would be accessed with flat instructions.)
template <class T>
using gptr = const T __attribute__((address_space(1)))*;
template <class T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return (gptr<T>)((uint64_t(hi) << 32) | lo);
}

// base (scalar registers) + uniform byte offset + the lane's 32-bit byte offset
template <class T>
__device__ __forceinline__ gptr<T> at(gptr<char> base, uint64_t uniform_bytes, uint32_t lane_bytes) {
  return (gptr<T>)(base + uniform_bytes + lane_bytes);
}

// 16-byte weight load; with STREAM the non-temporal hint (data used once).
template <bool STREAM>
__device__ __forceinline__ uint4 ld_w(gptr<uint4> p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const gptr<u32x4> q = (gptr<u32x4>)p;
  const u32x4 v = STREAM ? __builtin_nontemporal_load(q) : *q;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

// e4m3fn x 8 (two dwords) -> bf16 x 8 of code * scale: exact decode to fp32
// (v_cvt_pk_f32_fp8), one fp32 multiply by the 128x128 block scale, one RNE
// rounding to bf16. (v_cvt_scalef32_pk_bf16_fp8 would apply only the
// power-of-two exponent of a scale, which block scales are not.)
__device__ __forceinline__ bf16x8_t fp8x8_dequant(uint32_t w0, uint32_t w1, float s) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r0 = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w0, false) * s, bf16x2_t);
  const bf16x2_t r1 = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w0, true) * s, bf16x2_t);
  const bf16x2_t r2 = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w1, false) * s, bf16x2_t);
  const bf16x2_t r3 = __builtin_convertvector(__builtin_amdgcn_cvt_pk_f32_fp8(w1, true) * s, bf16x2_t);
  bf16x8_t r;
  r[0] = r0[0]; r[1] = r0[1]; r[2] = r1[0]; r[3] = r1[1];
  r[4] = r2[0]; r[5] = r2[1]; r[6] = r3[0]; r[7] = r3[1];
  return r;
}

// ------------------------------------------------------------------ MFMA kernel
// Stream-K split of the work: the iterations (tile, 128-deep K chunk) of the
// whole launch are cut into equal contiguous ranges, one per workgroup (at
// most kBfGrid for bf16 weights, kF8Grid for fp8: one resident workgroup per
// compute unit), so every workgroup streams the same number of weight bytes no
// matter how the tile count compares with the number of workgroups. A tile
// covered by one workgroup is finished in place; a tile cut by a range
// boundary leaves fp32 partial sums (in accumulator-register order) in the
// workspace, and ffn_fixup_kernel adds them in workgroup order and finishes
// the tile. No workgroup ever waits for another. When the launch has little
// work, fewer ranges are used (at least kSkMinChunks chunks each), so the
// partial sums stay small next to the weights streamed.
constexpr int kXcds = 8;                              // accelerator complex dies of MI355X
constexpr int kPartFloats = 4 * kMB * 16 * kWave;     // a bf16 workgroup's accumulators (64 KiB: 8 waves x 2 blocks)
constexpr int kSkMinChunks = 8;

// bf16 decode kernel (ffn_bf16_kernel): tiles of 64 activation rows x two N
// blocks for a workgroup of 8 waves, one workgroup per compute unit
constexpr int kBfBM = kBM / 2;                 // activation rows per tile
constexpr int kBfMB = kBfBM / 32;              // 32-row MFMA blocks per tile
constexpr int kBfWaves = 8;                    // waves per workgroup (one workgroup per CU)
constexpr int kBfThreads = kBfWaves * kWave;
constexpr int kBfNB = kBfWaves / 4;            // N blocks per tile
constexpr int kBfGrid = 256;                   // 1 resident workgroup x 256 CUs
static_assert(kBfThreads <= kMaxGemmThreads, "schedule scratch holds one entry per thread");
static_assert(kBfWaves * kBfMB * 16 * kWave <= kPartFloats, "a workgroup's accumulators fit a partial slot");
// [wave][block][quad q][lane][4 floats]: 1 KiB contiguous per wave access
__device__ __forceinline__ int bf_part_idx(int wv, int b, int q, int lane) {
  return (((wv * kBfMB + b) * 4 + q) * kWave + lane) * 4;
}

// Ranges used for a launch of `total` iterations: a multiple of the XCD count.
__device__ inline int sk_grid(int64_t total, int max_grid) {
  const int64_t g = total / kSkMinChunks / kXcds * kXcds;
  return int(max<int64_t>(kXcds, min<int64_t>(max_grid, g)));
}

__host__ __device__ inline int64_t sk_start(int b, int64_t total, int G) { return int64_t(b) * total / G; }

// Range whose span holds iteration i (the last one, if several start there).
__device__ inline int sk_owner(int64_t i, int64_t total, int G) {
  return int(((i + 1) * G + total - 1) / total) - 1;
}

// Partial slot of workgroup b: 0 for its first tile, 1 for its last.
__device__ inline float* sk_slot(float* parts, int b, int slot) {
  return parts + (size_t(b) * 2 + slot) * kPartFloats;
}

// Epilogue of 32-row block b of a tile (four consecutive output columns never
// straddle a 32-column block).
template <int KIND>
__device__ __forceinline__ void ffn_epilogue_block(const f32x16_t& acc, const Tile& tl, int b, const Sched& sh,
                                                   uint16_t* out, int n_out, int wv, int lr, int lh, bool oblk) {
  const int phys = sh.rowmap[b * 32 + lr];
  if (phys < 0) return;
  uint16_t* orow = out + act_off(phys, 0, n_out, oblk);
  if (KIND == kUp) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = silu_f(acc[4 * q + r]) * acc[4 * (q + 2) + r];
      const int col = tl.nt * 64 + 16 * wv + 8 * q + 4 * lh;
      *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
          make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = tl.nt * 128 + 32 * wv + 8 * q + 4 * lh;
      *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
          make_uint2(pack_bf16x2(acc[4 * q], acc[4 * q + 1]), pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3]));
    }
  }
}

template <int KIND, int NBMAX>
__device__ __forceinline__ void ffn_epilogue(const f32x16_t (&acc)[NBMAX], const Tile& tl, int nb, const Sched& sh,
                                             uint16_t* out, int n_out, int wv, int lr, int lh, bool oblk) {
#pragma unroll
  for (int b = 0; b < NBMAX; ++b)
    if (b < nb) ffn_epilogue_block<KIND>(acc[b], tl, b, sh, out, n_out, wv, lr, lh, oblk);
}

// NA accumulator tiles (16 floats per lane each) summed over the partials of
// ranges w_lo .. w_hi in range order; src(w) is the partial of range w
// (nullptr: an empty range, nothing to add) and idx(a, q) the offset of quad q
// of tile a in it. The loads of four ranges are in flight at a time.
template <int NA, class Src, class Idx>
__device__ __forceinline__ void sum_partials(f32x16_t (&acc)[NA], int w_lo, int w_hi, Src src, Idx idx) {
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[a][v] = 0.f;
  for (int w0 = w_lo; w0 <= w_hi; w0 += 4) {
    float4 ld[4][NA][4];
    const float* ps[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ps[k] = w0 + k <= w_hi ? src(w0 + k) : nullptr;
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ld[k][a][q] = ps[k] ? *reinterpret_cast<const float4*>(ps[k] + idx(a, q)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!ps[k]) continue;  // uniform
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[a][4 * q] += ld[k][a][q].x;
          acc[a][4 * q + 1] += ld[k][a][q].y;
          acc[a][4 * q + 2] += ld[k][a][q].z;
          acc[a][4 * q + 3] += ld[k][a][q].w;
        }
    }
  }
}

// Finishes the tiles of ffn_bf16_kernel cut by a stream-K range boundary:
// block (j, m * kBfMB + b) looks at the boundary between workgroups j and
// j+1; the first boundary inside a tile sums, for the tile's N block m and
// 32-row block b, its partials in workgroup order (one wave per 32 weight rows
// of the N block, i.e. the partials of the main kernel's waves 4 m .. 4 m + 3)
// and runs that block's epilogue.
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int ntn2 = (p.n_tiles_n + kBfNB - 1) / kBfNB;
  const int n_tiles = build_schedule(p, kBfBM, ntn2, false, sh);
  const int nchunks = p.K / kKC;
  const int64_t total = int64_t(n_tiles) * nchunks;
  const int j = blockIdx.x, m = blockIdx.y / kBfMB, b = blockIdx.y % kBfMB;
  const int G = sk_grid(total, kBfGrid);
  if (j + 1 >= G) return;  // uniform: boundaries lie between ranges 0 .. G-1
  const int64_t ib = sk_start(j + 1, total, G);
  if (ib <= 0 || ib >= total || ib % nchunks == 0) return;  // not inside a tile
  const int t = int(ib / nchunks);
  if (j > 0 && sk_start(j, total, G) > int64_t(t) * nchunks) return;  // an earlier boundary owns this tile
  Tile tl = decode_tile(p, kBfBM, ntn2, sh, t);
  if (b * 32 >= tl.nrows || kBfNB * tl.nt + m >= p.n_tiles_n) return;  // uniform: no rows / no such N block
  build_rowmap(p, tl, kBfBM, sh);
  const int b_lo = sk_owner(int64_t(t) * nchunks, total, G);
  const int b_hi = sk_owner(int64_t(t + 1) * nchunks - 1, total, G);
  f32x16_t acc[1];
  sum_partials(
      acc, b_lo, b_hi,
      [&](int w) -> const float* {
        const int64_t s0 = sk_start(w, total, G), s1 = sk_start(w + 1, total, G);
        return s0 < s1 ? sk_slot(const_cast<float*>(parts), w, int(s0 / nchunks) == t ? 0 : 1) : nullptr;
      },
      [&](int, int q) { return bf_part_idx(4 * m + wv, b, q, lane); });
  tl.nt = kBfNB * tl.nt + m;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  ffn_epilogue_block<KIND>(acc[0], tl, b, sh, out, p.n_out, wv, lr, lh, p.out_blk);
}

// ------------------------------------------------------------------ wide-tile kernel
// Groups with many rows (prefill, and decode with few experts per GPU) are
// compute-heavy: a weight block is used by hundreds of rows, so it pays to
// stage it once in LDS and reuse every operand fragment several times from
// registers. Tile = 256 weight rows x 256 activation rows; each of the 4 waves
// owns 64 weight rows (up: 32 gate rows and the 32 matching up rows, so the
// SwiGLU pairs meet in one lane) against all 256 activation rows, i.e. a
// 64 x 256 accumulator block (2 x 8 MFMA 32x32 tiles, 256 accumulator
// registers; one wave per SIMD). Per 16-deep step a wave reads 2 weight and
// up to 8 activation fragments from LDS for up to 16 MFMAs.
//
// Data path: global -> LDS directly (global_load_lds, 16 bytes per lane; lane
// l of a load writes bytes [16 l, 16 l + 16) of the 1 KiB the wave's load
// covers), in kWK-deep stages through a ring of kWStages LDS buffers (128 KiB
// in all), so all but one stage are in flight while one is multiplied, and no
// registers hold data in transit. Each wave waits for its own loads of a stage
// (vmcnt) before the barrier that publishes it; the barrier sits before the
// last 16-deep step of each stage, whose fragments are already in registers,
// so the fragment reads of the next stage overlap its MFMAs.
// LDS: 64 banks of 4 bytes, a 128-bit access is served 16 lanes at a time.
// A row holds one stage of one operand row (kWK bf16, kWSlots 16-byte slots)
// and slot s of row r holds column s ^ ((r / (16 / kWSlots)) % kWSlots): the 16
// rows a fragment load reads together fall on 16 distinct 16-byte bank
// groups. The swizzle is applied on the global side (each lane fetches the
// column its LDS slot holds).
// Activation blocks past the tile's rows are not multiplied (NB), and their
// loads are limited to what keeps every wave's load count equal.
// Tiles are ordered (group, blocked row/N tiles) and handed out so that the 32
// workgroups of one XCD take consecutive tiles, which share operand slabs in
// that XCD's L2.
constexpr int kWStages = 128 / kWK;     // LDS ring depth (the ring holds 128 KiB)
constexpr int kWSlots = kWK / 8;        // 16-byte slots per LDS row
constexpr int kWRowsPerLoad = 64 / kWSlots;  // rows one 1 KiB wave load covers
constexpr int kWStage = kWN * kWK;      // elements of one operand per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of 16 bytes per lane (lane l writes bytes [16 l, 16 l +
// 16) of the wave's KiB at lds), from scalar base + the lane's 32-bit offset:
// global_load_lds as inline assembly, so that the compiler's wait-count
// analysis does not see it. (With an LDS-writing global load outstanding that
// analysis waits for every vector-memory op before the next use of any loaded
// register, which would cap the prefetch at one stage.) The caller's own
// counted waits must cover it; ops the analysis does not know of only make
// its waits longer, since the count retires in order.
__device__ __forceinline__ void lds_dma16_untracked(gptr<char> base, uint32_t lane_off, const void* lds) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_ptr_t)lds);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(base), "{m0}"(l) : "memory");
}

// Raw buffer resource over the 4 GiB from a wave-uniform base (scalar
// registers): a buffer load addresses base + scalar offset + the lane's 32-bit
// offset + an immediate, so no per-lane 64-bit address is held in registers.
// (num_records is the maximum: the offsets are our own and stay in range.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  // (readfirstlane returns a signed int: each half goes through uint32_t, or
  // widening would sign-extend the low half over the high one)
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  const uint64_t u = (uint64_t(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), short(0), -1, 0x00020000);
}

// s_waitcnt immediate: wait until at most n vector-memory ops are outstanding
// and no LDS op is (gfx9 encoding: vmcnt[3:0], expcnt[6:4] (7 = no wait),
// lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }
// s_waitcnt operand: at most n vector-memory ops outstanding, LDS/scalar count not waited for
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// The ring buffers are separate LDS objects, and the stage loop is unrolled by
// the ring depth so every load and fragment read names its buffer statically:
// the compiler can then see that a read does not touch the buffers still being
// filled and does not wait for those loads.
struct WideLds {
  uint16_t* w[4];
  uint16_t* x[4];
};

// One wide tile's accumulators: 4 waves x (gate/up or two output halves) x 8
// activation blocks x 16 registers x 64 lanes.
constexpr int kWidePart = 4 * 2 * 8 * 16 * kWave;
// [wave][a][block][quad q][lane][4 floats]: registers 4q..4q+3 of one
// accumulator tile, 16 bytes per lane, 1 KiB contiguous per wave access
__device__ __forceinline__ int wide_part_idx(int wv, int a, int b, int q, int lane) {
  return ((((wv * 2 + a) * 8 + b) * 4 + q) * kWave + lane) * 4;
}

// Epilogue of one 32-row activation block b of a wide tile from its two
// accumulator tiles (up: gate and up rows of the same h columns; down: the two
// 32-row halves of the wave's 64 output columns).
template <int KIND>
__device__ __forceinline__ void wide_epilogue_block(const GemmArgs& p, const Tile& tl, const Sched& sh, int b,
                                                    const f32x16_t& a0, const f32x16_t& a1, int wv, int lr, int lh) {
  const int phys = sh.rowmap[32 * b + lr];
  if (phys < 0) return;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  const bool oblk = p.out_blk;
  uint16_t* orow = out + act_off(phys, 0, p.n_out, oblk);
  if (KIND == kUp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = silu_f(a0[4 * q + r]) * a1[4 * q + r];
      const int col = tl.nt * 128 + 32 * wv + 8 * q + 4 * lh;
      *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
          make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
    }
  } else {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const f32x16_t& ac = a ? a1 : a0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = tl.nt * 256 + 64 * wv + 32 * a + 8 * q + 4 * lh;
        *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
            make_uint2(pack_bf16x2(ac[4 * q], ac[4 * q + 1]), pack_bf16x2(ac[4 * q + 2], ac[4 * q + 3]));
      }
    }
  }
}

// Stages [s_begin, s_end) of one wide tile (a multiple of the ring depth).
// part == nullptr: the range is the whole tile, run the epilogue; else leave
// the fp32 accumulators in part for ffn_wide_fixup_kernel.
template <int KIND, bool PACKED, int NB>
__device__ __forceinline__ void wide_tile(const GemmArgs& p, const Tile& tl, const Sched& sh, const WideLds& L,
                                          int s_begin, int s_end, float* __restrict__ part) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int last = s_end - 1;
  const uint16_t* A = static_cast<const uint16_t*>(pick(tl.shared, p.sh_a, p.a));
  const uint16_t* W = static_cast<const uint16_t*>(pick(tl.shared, p.sh_w, p.w));

  // Load q of wave wv covers tile rows kWRowsPerLoad (4 q + wv) + lane /
  // kWSlots, LDS slot lane % kWSlots, i.e. global column
  // cg = (lane % kWSlots) ^ swizzle(row). WL loads per wave per stage for the
  // weights; XL for the activations, enough for NB blocks (rows past the
  // tile's rows re-read row 0 of the tile into rows nobody multiplies).
  constexpr int WL = kWN / kWRowsPerLoad / 4;
  constexpr int XL = (NB * 32 / kWRowsPerLoad + 3) / 4;
  constexpr int P = WL + XL;  // loads per wave per stage
  const int lrow = lane / kWSlots;
  auto col_of = [&](int row) { return (lane % kWSlots) ^ ((row / (16 / kWSlots)) % kWSlots); };
  const bool ablk = pick(tl.shared, p.sh_a_blk, p.a_blk);
  const size_t xstep = ablk ? 512 : kWK;  // elements from one stage of a row to the next
  const uint16_t* xg[XL];
  const bool gat = p.a_rows != nullptr && !tl.shared;  // input rows gathered from a
  const int* amap = gat ? sh.arow : sh.rowmap;
  const int phys0 = amap[0];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int row = kWRowsPerLoad * (4 * q + wv) + lrow;
    const int phys = row < NB * 32 ? amap[row] : -1;
    const int pr = phys >= 0 ? phys : phys0;
    // (columns 8 cg .. 8 cg + 7 of stage 0 lie inside the first 32-column block)
    xg[q] = A + (ablk ? blk_row_base(pr, p.K) : size_t(pr) * p.K) + col_of(row) * 8;
  }
  const uint16_t* wg[WL];
#pragma unroll
  for (int q = 0; q < WL; ++q) {
    const int R = kWRowsPerLoad * (4 * q + wv) + lrow;  // tile weight row
    const int cg = col_of(R);
    if constexpr (!PACKED) {
      int row;
      if (KIND == kUp) row = ((R >> 5) & 1 ? p.n_out : 0) + tl.nt * 128 + 32 * (R >> 6) + (R & 31);
      else row = tl.nt * 256 + R;
      wg[q] = W + (size_t(tl.we) * p.n_w_rows + row) * p.K + cg * 8;
    } else {
      // the 16-byte piece of the packed layout [g][ntp][c][w][i][lane] that holds
      // this row's columns [8 cg, 8 cg + 8) of stage 0 (k = 128 c + 64 (i / 4) +
      // 32 (lane / 32) + 8 (i % 4))
      int ntp, wdec, lrp;
      if (KIND == kUp) {
        const int j = tl.nt * 128 + 32 * (R >> 6) + (R & 31);  // h column
        ntp = j >> 6;
        wdec = (j & 63) >> 4;
        lrp = ((R >> 5) & 1) * 16 + (j & 15);
      } else {
        const int row = tl.nt * 256 + R;
        ntp = row >> 7;
        wdec = (row & 127) >> 5;
        lrp = row & 31;
      }
      const int nchunks = p.K / kKC;
      const size_t piece = ((size_t(tl.we) * p.n_tiles_n + ntp) * nchunks * 4 + wdec) * 8 * kWave +
                           (cg & 3) * kWave + ((cg >> 2) & 1) * 32 + lrp;
      wg[q] = W + piece * 8;
    }
  }
  // element offset of stage kt relative to stage 0 (packed: the stage's first
  // column kb = kWK kt sets the chunk, the load's upper half and the lane half)
  auto woff = [&](int kt) -> size_t {
    if constexpr (PACKED) {
      const int kb = kWK * kt;
      return (size_t(kb >> 7) * 4 * 8 * kWave + size_t((kb >> 6) & 1) * 4 * kWave + size_t((kb >> 5) & 1) * 32) * 8;
    } else {
      return size_t(kt) * kWK;
    }
  };
#define MOE_WIDE_ISSUE(KT_, SLOT_)                                                                          \
  {                                                                                                         \
    const size_t wo_ = woff(KT_), xo_ = size_t(KT_) * xstep;                                                \
    _Pragma("unroll") for (int q = 0; q < WL; ++q)                                                          \
      __builtin_amdgcn_global_load_lds(wg[q] + wo_, (lds_ptr_t)(L.w[SLOT_] + (4 * q + wv) * 512), 16, 0, 0);  \
    _Pragma("unroll") for (int q = 0; q < XL; ++q)                                                          \
      __builtin_amdgcn_global_load_lds(xg[q] + xo_, (lds_ptr_t)(L.x[SLOT_] + (4 * q + wv) * 512), 16, 0, 0);  \
  }

  f32x16_t acc[2][NB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const int fsw = (lr / (16 / kWSlots)) % kWSlots;
  const int arow0 = (64 * wv + lr) * kWK, arow1 = (64 * wv + 32 + lr) * kWK;
  // two fragment sets: all ten reads of step s+1 are issued at the start of
  // step s, so they have the whole step to land
  bf16x8_t fa[2][2], fb[2][NB];
#define MOE_WIDE_FRAGS(SET_, WBUF_, XBUF_, S_)                                                              \
  {                                                                                                         \
    const int col_ = ((2 * (S_) + lh) ^ fsw) * 8;                                                           \
    fa[SET_][0] = *reinterpret_cast<const bf16x8_t*>((WBUF_) + arow0 + col_);                               \
    fa[SET_][1] = *reinterpret_cast<const bf16x8_t*>((WBUF_) + arow1 + col_);                               \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                          \
        fb[SET_][b] = *reinterpret_cast<const bf16x8_t*>((XBUF_) + (32 * b + lr) * kWK + col_);             \
  }
#define MOE_WIDE_MFMAS(SET_)                                                                                \
  _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                          \
    acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET_][0], fb[SET_][b], acc[0][b], 0, 0, 0);      \
    acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET_][1], fb[SET_][b], acc[1][b], 0, 0, 0);      \
  }

  // prologue: stages 0 .. kWStages-2 in flight, wait for stage 0
  constexpr int NS = kWK / 16;  // 16-deep MFMA steps per stage
#pragma unroll
  for (int st = 0; st < kWStages - 1; ++st) MOE_WIDE_ISSUE(min(s_begin + st, last), st)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((kWStages - 2) * P));
  __builtin_amdgcn_s_barrier();
  MOE_WIDE_FRAGS(0, L.w[0], L.x[0], 0)

  // One stage (two 16-deep steps); J = stage % kWStages is a literal in each
  // expansion. While LDS-DMA loads are outstanding the compiler waits for all
  // LDS reads (lgkmcnt(0)) before using any fragment, so the reads are placed
  // where that wait finds them done: the step-1 fragments are read in the
  // middle of step 0's MFMAs, the next stage's step-0 fragments right after
  // the barrier, ahead of step 1's MFMAs.
#define MOE_WIDE_MFMA_RANGE(SET_, B0_, B1_)                                                                 \
  _Pragma("unroll") for (int b = (B0_); b < (B1_); ++b) {                                                   \
    acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET_][0], fb[SET_][b], acc[0][b], 0, 0, 0);      \
    acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET_][1], fb[SET_][b], acc[1][b], 0, 0, 0);      \
  }
#define MOE_WIDE_STAGE(J_, KT_)                                                                             \
  {                                                                                                         \
    MOE_WIDE_MFMA_RANGE(0, 0, (NB + 1) / 2)                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_WIDE_FRAGS(1, L.w[J_], L.x[J_], 1)                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_WIDE_MFMA_RANGE(0, (NB + 1) / 2, NB)                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    /* the stage kWStages-1 ahead goes into the buffer the previous stage used  \
       (everyone finished reading it before the previous barrier); past the    \
       end a harmless repeat */                                                                             \
    MOE_WIDE_ISSUE(min((KT_) + kWStages - 1, last), ((J_) + kWStages - 1) % kWStages)                       \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    /* this wave's loads of the next stage are done (later stages may still be \
       in flight); the barrier makes every wave's part visible */                                          \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((kWStages - 2) * P));                                       \
    __builtin_amdgcn_s_barrier();                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_WIDE_FRAGS(0, L.w[((J_) + 1) % kWStages], L.x[((J_) + 1) % kWStages], 0)                            \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_WIDE_MFMA_RANGE(1, 0, NB)                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
  }
  static_assert(NS == 2, "the stage body is written for two 16-deep steps");
  // the stage count is a multiple of kWStages (ranges are whole 128-deep chunks)
  for (int kt = s_begin; kt < s_end; kt += kWStages) {
    MOE_WIDE_STAGE(0, kt)
    MOE_WIDE_STAGE(1, kt + 1)
    if constexpr (kWStages == 4) {
      MOE_WIDE_STAGE(2, kt + 2)
      MOE_WIDE_STAGE(3, kt + 3)
    }
  }
#undef MOE_WIDE_STAGE
#undef MOE_WIDE_ISSUE
#undef MOE_WIDE_FRAGS
#undef MOE_WIDE_MFMAS
#undef MOE_WIDE_MFMA_RANGE
  // no load may still be writing LDS when the next tile reuses the buffers
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();

  if (part == nullptr) {
#pragma unroll
    for (int b = 0; b < NB; ++b) wide_epilogue_block<KIND>(p, tl, sh, b, acc[0][b], acc[1][b], wv, lr, lh);
  } else {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; v += 4)
          *reinterpret_cast<float4*>(part + wide_part_idx(wv, a, b, v / 4, lane)) =
              make_float4(acc[a][b][v], acc[a][b][v + 1], acc[a][b][v + 2], acc[a][b][v + 3]);
  }
}

// Work split of the wide kernel (kWideGrid workgroups, one per compute unit):
// whole tiles in full rounds, tile r * kWideGrid + (XCD-blocked slot of the
// workgroup), so the 32 workgroups of an XCD work on 32 consecutive tiles of
// the blocked order; then the last n_tiles % kWideGrid tiles are split along
// K into S equal chunk ranges each (S as large as the idle workgroups allow,
// at least kWideMinChunks chunks per range), so a launch with few tiles (a
// decode batch with few experts per GPU) still keeps the compute units busy.
// A split leaves fp32 partials (one slot per workgroup); ffn_wide_fixup_kernel
// adds the S partials of a tile in split order and runs the epilogue.
constexpr int kWideMinChunks = 4;

struct WideSplit {
  int full;   // tiles done whole, in full rounds
  int rem;    // tiles split along K
  int S;      // ranges per split tile
};

__device__ inline WideSplit wide_split(int n_tiles, int nch) {
  WideSplit w;
  w.full = n_tiles / kWideGrid * kWideGrid;
  w.rem = n_tiles - w.full;
  w.S = w.rem ? max(1, min(kWideGrid / w.rem, nch / kWideMinChunks)) : 1;
  return w;
}

template <int KIND, bool PACKED>
__global__ __launch_bounds__(kGemmThreads, 1) void ffn_wide_kernel(GemmArgs p, float* __restrict__ parts) {
  __shared__ Sched sh;
  constexpr int kExtra = kWStages == 4 ? kWStage : 8;  // buffers 2 and 3 exist with a 4-deep ring only
  __shared__ __attribute__((aligned(1024))) uint16_t w0[kWStage], w1[kWStage], w2[kExtra], w3[kExtra];
  __shared__ __attribute__((aligned(1024))) uint16_t x0[kWStage], x1[kWStage], x2[kExtra], x3[kExtra];
  const WideLds L = {{w0, w1, w2, w3}, {x0, x1, x2, x3}};
  const int ntn = KIND == kUp ? p.n_out / 128 : p.n_out / 256;
  const int n_tiles = build_schedule(p, kWM, ntn, true, sh);
  const int nch = p.K / kKC;  // 128-deep chunks per tile
  constexpr int SPC = kKC / kWK;  // stages per chunk
  const WideSplit ws = wide_split(n_tiles, nch);
  const int slot = int(blockIdx.x % kXcds) * (kWideGrid / kXcds) + int(blockIdx.x / kXcds);
  auto run = [&](int t, int c_begin, int c_end, float* part) __attribute__((always_inline)) {
    const Tile tl = decode_tile<true>(p, kWM, ntn, sh, t);
    build_rowmap(p, tl, kWM, sh, true);
    const int sb = c_begin * SPC, se = c_end * SPC;
    switch ((tl.nrows + 31) / 32) {
      case 1: wide_tile<KIND, PACKED, 1>(p, tl, sh, L, sb, se, part); break;
      case 2: wide_tile<KIND, PACKED, 2>(p, tl, sh, L, sb, se, part); break;
      case 3: wide_tile<KIND, PACKED, 3>(p, tl, sh, L, sb, se, part); break;
      case 4: wide_tile<KIND, PACKED, 4>(p, tl, sh, L, sb, se, part); break;
      case 5: wide_tile<KIND, PACKED, 5>(p, tl, sh, L, sb, se, part); break;
      case 6: wide_tile<KIND, PACKED, 6>(p, tl, sh, L, sb, se, part); break;
      case 7: wide_tile<KIND, PACKED, 7>(p, tl, sh, L, sb, se, part); break;
      default: wide_tile<KIND, PACKED, 8>(p, tl, sh, L, sb, se, part); break;
    }
    __syncthreads();  // rowmap is rewritten by the next tile
  };
  for (int t = slot; t < ws.full; t += kWideGrid) run(t, 0, nch, nullptr);
  const int u = int(blockIdx.x);  // split unit: tile full + u / S, range u % S
  if (ws.rem && u < ws.rem * ws.S) {
    const int t = ws.full + u / ws.S, k = u % ws.S;
    if (ws.S == 1) {
      run(t, 0, nch, nullptr);
    } else {
      run(t, k * nch / ws.S, (k + 1) * nch / ws.S, parts + size_t(u) * kWidePart);
    }
  }
}

// Finishes the split wide tiles: block (i, b) sums the S partials of split
// tile i for activation block b in split order and runs its epilogue.
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_wide_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int ntn = KIND == kUp ? p.n_out / 128 : p.n_out / 256;
  const int n_tiles = build_schedule(p, kWM, ntn, true, sh);
  const int nch = p.K / kKC;
  const WideSplit ws = wide_split(n_tiles, nch);
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= ws.rem || ws.S == 1) return;  // uniform
  const int t = ws.full + i;
  const Tile tl = decode_tile<true>(p, kWM, ntn, sh, t);
  if (b * 32 >= tl.nrows) return;  // uniform: no rows in this block
  build_rowmap(p, tl, kWM, sh);
  // the S partials of each accumulator tile in split order, four in flight at a time
  f32x16_t acc[2];
  sum_partials(
      acc, 0, ws.S - 1, [&](int k) -> const float* { return parts + size_t(i * ws.S + k) * kWidePart; },
      [&](int a, int q) { return wide_part_idx(wv, a, b, q, lane); });
  wide_epilogue_block<KIND>(p, tl, sh, b, acc[0], acc[1], wv, lr, lh);
}

// ------------------------------------------------------------------ bf16 decode kernel
// bf16 weights, decode-shaped groups: stream-K ranges over tiles of 64
// activation rows x two adjacent N blocks (256 weight rows) for a workgroup of
// 8 waves, one per compute unit (each wave 32 weight rows of one block; up: 16
// gate rows and the 16 matching up rows), the activations staged by
// LDS DMA and the weights
// loaded straight into registers (each lane 8 16-byte pieces of its weight row
// per chunk). Three chunks are in flight per workgroup (three LDS activation
// buffers, a three-deep weight register ring): all loads of chunk c+2 are
// issued at the top of chunk c, right after the barrier, and the wait at the
// top of a chunk leaves the next chunk's loads outstanding.
// A group with one row tile has its N tiles next to each other in the
// schedule, and they read the same activation rows: a workgroup streams such a
// run of tiles as one sequence of chunks, so the loads run ahead across tile
// boundaries instead of draining at every tile (with K = 2048 a tile is only
// 16 chunks); each tile's epilogue is issued as soon as its last chunk is
// multiplied.

// Tiles tl.nt .. tl.nt + n - 1 of one group and row tile, iterations
// [it_begin, it_end) of the run (iteration k * nchunks + c is chunk c of its
// tile k). A tile is 64 activation rows x two N blocks; wave w owns weight
// rows 32 (w % 4) .. + 31 of N block 2 tile + w / 4 (past the group's last
// block a wave repeats it and its results are discarded), so each staged
// activation chunk feeds 256 weight rows. The first / last tile leave fp32 partials in part_first /
// part_last when split (else nullptr: their epilogue runs here).
template <int KIND, bool PACKED, int NB, bool STREAM>
__device__ __forceinline__ void bf_run(const GemmArgs& p, const Tile& tl, int n, const Sched& sh,
                                       uint16_t* __restrict__ x0, uint16_t* __restrict__ x1,
                                       uint16_t* __restrict__ x2, int it_begin, int it_end,
                                       float* __restrict__ part_first, float* __restrict__ part_last) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar
  const int wq = wv & 3;   // the wave's 32 weight rows of its N block
  const int wg = wv >> 2;  // the wave's N block in the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nchunks = p.K / kKC;
  const int last = it_end - 1;
  // N block of the run's tile k for this wave
  const int nb0 = __builtin_amdgcn_readfirstlane(kBfNB * tl.nt + wg);
  const int nb_max = __builtin_amdgcn_readfirstlane(p.n_tiles_n - 1);
  auto nbof = [&](int k) { return min(nb0 + kBfNB * k, nb_max); };

  // weights: this lane's row of N block 0; piece j of chunk C covers
  // k = 128 C + 64 (j / 4) + 32 lh + 8 (j % 4)
  const uint16_t* W = static_cast<const uint16_t*>(pick(tl.shared, p.sh_w, p.w));
  int wrow;
  if (KIND == kUp) {
    const int j = 16 * wq + (lr & 15);
    wrow = lr < 16 ? j : p.n_out + j;
  } else {
    wrow = 32 * wq + lr;
  }
  // uniform base (the expert's block) + the lane's loop-invariant byte offset
  // (an expert's weights span less than 4 GiB)
  gptr<char> wbase;
  uint32_t woff;
  if constexpr (PACKED) {
    wbase = uniform_ptr(reinterpret_cast<const char*>(W) + size_t(tl.we) * p.n_tiles_n * nchunks * 4 * 8 * kWave * 16);
    woff = uint32_t(wq * 8 * kWave + lane) * 16u;
  } else {
    wbase = uniform_ptr(reinterpret_cast<const char*>(W + size_t(tl.we) * p.n_w_rows * p.K));
    woff = uint32_t(wrow * p.K + 32 * lh) * 2u;
  }
  // iteration (tile k, chunk C), piece j: packed, block nb's chunks follow each
  // other; row-major, block nb's rows are 64 (gate and up) or 128 rows below
  // block 0's
  const uint64_t tstep = uint64_t(KIND == kUp ? 64 : 128) * p.K * 2;
  auto wpiece = [&](int k, int C, int j) -> gptr<uint4> {
    const int nb = nbof(k);
    if constexpr (PACKED) {
      return at<uint4>(wbase, ((uint64_t(nb) * nchunks + C) * 4 * 8 + j) * kWave * 16, woff);
    } else {
      return at<uint4>(wbase, nb * tstep + uint64_t(C) * kKC * 2 + (j >> 2) * 128 + (j & 3) * 16, woff);
    }
  };

  // activations: load q of this wave stages tile rows 4 (8 q + wv) .. + 3
  constexpr int XL = NB * 8 / kBfWaves;  // 1 KiB loads per wave per chunk
  const uint16_t* A = static_cast<const uint16_t*>(pick(tl.shared, p.sh_a, p.a));
  const bool ablk = pick(tl.shared, p.sh_a_blk, p.a_blk);
  const size_t xstep = ablk ? size_t(4) * 512 : size_t(kKC);  // elements from one chunk of a row to the next
  // per-lane byte offsets from the tile's first row (a tile's rows lie in one
  // expert's region, which the host keeps below 2^31 elements); gathered rows
  // from a's start (the host keeps a below 2^32 bytes)
  const bool gat = p.a_rows != nullptr && !tl.shared;
  const int* amap = gat ? sh.arow : sh.rowmap;
  const int phys0 = amap[0];
  const size_t xbase = gat ? 0 : ablk ? blk_row_base(phys0, p.K) : size_t(phys0) * p.K;
  const gptr<char> xb = uniform_ptr(reinterpret_cast<const char*>(A + xbase));
  uint32_t xoff[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int r = 4 * (kBfWaves * q + wv) + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);  // column piece this lane's LDS slot holds
    const int phys = amap[r];
    const int pr = phys >= 0 ? phys : phys0;  // rows past the tile feed only discarded columns
    xoff[q] = uint32_t((ablk ? blk_row_base(pr, p.K) + size_t(c >> 2) * 512 + (c & 3) * 8 : size_t(pr) * p.K + c * 8) -
                       xbase) * 2u;
  }

  f32x16_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));

  uint4 w0[8], w1[8], w2[8];  // weight ring
#define MOE_BF_LOADS(I_, XBUF_, WR_)                                                                          \
  {                                                                                                         \
    const int k_ = (I_) / nchunks, c_ = (I_) - k_ * nchunks;                                                \
    const size_t xo_ = size_t(c_) * xstep;                                                                  \
    _Pragma("unroll") for (int q = 0; q < XL; ++q)                                                          \
      __builtin_amdgcn_global_load_lds(at<void>(xb, xo_ * 2, xoff[q]), (lds_ptr_t)((XBUF_) + (kBfWaves * q + wv) * 512), 16, 0, 0); \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) WR_[j] = ld_w<STREAM>(wpiece(k_, c_, j));                 \
  }
  // this wave's loads of the chunk have landed (only the next chunk's, XL + 8
  // ops, and epilogue stores issued after them may be outstanding: loads
  // retire in order, so at most over-waiting); after the barrier every wave's
  // staged rows are visible and nobody still reads the buffer the next loads
  // overwrite
#define MOE_BF_SYNC()                                                                                       \
  __builtin_amdgcn_sched_barrier(0);                                                                        \
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(XL + 8));                                                     \
  __builtin_amdgcn_s_barrier();                                                                             \
  __builtin_amdgcn_sched_barrier(0);
#define MOE_BF_CHUNK(XBUF_, WR_)                                                                            \
  _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                           \
    const int cl_ = 8 * (j >> 2) + 4 * lh + (j & 3);                                                        \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                        \
      const int rr_ = b * 32 + lr;                                                                          \
      const bf16x8_t bv_ = *reinterpret_cast<const bf16x8_t*>((XBUF_) + rr_ * kKC + ((cl_ ^ (rr_ & 15)) * 8)); \
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, WR_[j]), bv_, acc[b], 0, 0, 0); \
    }                                                                                                       \
  }
  // after iteration I_: if it ends its tile, the tile's epilogue (or partial
  // sums) and fresh accumulators
#define MOE_BF_FINISH(I_)                                                                                   \
  {                                                                                                         \
    const int k_ = (I_) / nchunks;                                                                          \
    if ((I_) - k_ * nchunks == nchunks - 1 || (I_) == last) { /* uniform */                                 \
      float* part_ = k_ == 0 ? part_first : (k_ == n - 1 ? part_last : nullptr);                            \
      if (part_ == nullptr) {                                                                               \
        Tile tk_ = tl;                                                                                      \
        tk_.nt = kBfNB * (tl.nt + k_) + wg;                                                                 \
        if (tk_.nt < p.n_tiles_n) ffn_epilogue<KIND, NB>(acc, tk_, NB, sh, out, p.n_out, wq, lr, lh, p.out_blk); \
      } else {                                                                                              \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                      \
          _Pragma("unroll") for (int v = 0; v < 16; v += 4)                                                 \
            *reinterpret_cast<float4*>(part_ + bf_part_idx(wv, b, v / 4, lane)) =                           \
                make_float4(acc[b][v], acc[b][v + 1], acc[b][v + 2], acc[b][v + 3]);                        \
      }                                                                                                     \
      _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                        \
        _Pragma("unroll") for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;                                     \
    }                                                                                                       \
  }
  // iteration I_ in slot (XA_, WA_); loads iteration I_ + 2 into the slot two ahead (XN_, WN_)
#define MOE_BF_STEP(I_, XA_, WA_, XN_, WN_)                                                                 \
  {                                                                                                         \
    MOE_BF_SYNC()                                                                                           \
    MOE_BF_LOADS(min((I_) + 2, last), XN_, WN_) /* past the end a harmless repeat */                        \
    MOE_BF_CHUNK(XA_, WA_)                                                                                  \
    MOE_BF_FINISH(I_)                                                                                       \
  }

  MOE_BF_LOADS(it_begin, x0, w0)
  MOE_BF_LOADS(min(it_begin + 1, last), x1, w1)
  // (no exit in the middle of the three-chunk body: the accumulators would
  // need a second copy at the exit)
  int it = it_begin;
  for (; it + 3 <= it_end; it += 3) {
    MOE_BF_STEP(it, x0, w0, x2, w2)
    MOE_BF_STEP(it + 1, x1, w1, x0, w0)
    MOE_BF_STEP(it + 2, x2, w2, x1, w1)
  }
  if (it + 1 == it_end) {
    MOE_BF_STEP(it, x0, w0, x2, w2)
  } else if (it + 2 == it_end) {
    MOE_BF_STEP(it, x0, w0, x2, w2)
    MOE_BF_STEP(it + 1, x1, w1, x0, w0)
  }
#undef MOE_BF_STEP
#undef MOE_BF_FINISH
#undef MOE_BF_LOADS
#undef MOE_BF_SYNC
#undef MOE_BF_CHUNK
  // no load may still be writing LDS when the next run reuses the buffers
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
}

// Stream-K over (tile, chunk) iterations; ffn_fixup_kernel finishes the split
// tiles. XCD-aware range order: workgroups are dispatched round-robin over
// the 8 XCDs, so of G ranges, range r goes to workgroup (r % (G / 8)) * 8 +
// r / (G / 8); consecutive
// ranges (the N tiles of one expert, which share its activation rows) then run
// on one XCD and its L2 fetches those rows once.
template <int KIND, bool PACKED>
__global__ __launch_bounds__(kBfThreads, 1) void ffn_bf16_kernel(GemmArgs p, float* __restrict__ parts) {
  __shared__ Sched sh;
  __shared__ __attribute__((aligned(1024))) uint16_t x0[kBfBM * kKC], x1[kBfBM * kKC], x2[kBfBM * kKC];
  const int ntn2 = (p.n_tiles_n + kBfNB - 1) / kBfNB;
  const int n_tiles = build_schedule<kBfThreads>(p, kBfBM, ntn2, false, sh);
  const int nchunks = p.K / kKC;
  const int64_t total = int64_t(n_tiles) * nchunks;
  const int G = sk_grid(total, kBfGrid);
  if (int(blockIdx.x) >= G) return;  // uniform
  const int rng = int(blockIdx.x % kXcds) * (G / kXcds) + int(blockIdx.x / kXcds);
  const int64_t i0 = sk_start(rng, total, G), i1 = sk_start(rng + 1, total, G);
  if (i0 >= i1) return;  // uniform
  const int t_first = int(i0 / nchunks), t_last = int((i1 - 1) / nchunks);
  for (int t = t_first; t <= t_last;) {
    const Tile tl = decode_tile(p, kBfBM, ntn2, sh, t);
    build_rowmap<kBfThreads>(p, tl, kBfBM, sh, true);
    // a run: with one row tile the group's next tiles are its next N tiles
    // (same activation rows)
    const int n = tl.mtiles == 1 ? min(t_last - t + 1, ntn2 - tl.nt) : 1;
    const int64_t t0 = int64_t(t) * nchunks;
    const int it_begin = int(max<int64_t>(i0 - t0, 0));
    const int it_end = int(min<int64_t>(i1 - t0, int64_t(n) * nchunks));
    // a split tile leaves partials in the workgroup's slot (0 for its first tile, 1 for its last)
    const bool split_first = it_begin > 0 || (n == 1 && it_end < nchunks);
    const bool split_last = it_end < n * nchunks;
    float* part_first = split_first ? sk_slot(parts, rng, t == t_first ? 0 : 1) : nullptr;
    float* part_last = n == 1 ? part_first : (split_last ? sk_slot(parts, rng, 1) : nullptr);
    auto run = [&](auto stream_tag) __attribute__((always_inline)) {
      constexpr bool ST = decltype(stream_tag)::value;
      if (tl.nrows <= 32) bf_run<KIND, PACKED, 1, ST>(p, tl, n, sh, x0, x1, x2, it_begin, it_end, part_first, part_last);
      else bf_run<KIND, PACKED, 2, ST>(p, tl, n, sh, x0, x1, x2, it_begin, it_end, part_first, part_last);
    };
    if (tl.mtiles == 1) run(std::true_type{});
    else run(std::false_type{});
    __syncthreads();  // rowmap is rewritten by the next run
    t += n;
  }
}

// ------------------------------------------------------------------ fp8 kernel
// fp8 e4m3 weights, decode-shaped groups (W8A16). A tile is 96 activation
// rows x four adjacent N blocks (up: 4 x 64 h columns; down: 4 x 128 output
// columns), i.e. 512 weight rows, for a workgroup of 8 waves (one per compute
// unit, two waves per SIMD): wave w owns rows 32 (w % 4) .. + 31 of N blocks
// 2 (w / 4) + a (sub-blocks a = 0, 1). Every activation chunk staged in LDS so
// feeds 512 weight rows: at ~100 rows per expert the activation re-reads,
// which would otherwise rival the fp8 weight bytes, are three eighths of them.
// 96 rows (3 MFMA blocks) keep the accumulators (96 registers) and a two-deep
// weight ring (64) inside one wave's registers at two waves per SIMD.
// Weights stream from HBM straight into the register ring (each lane 64
// contiguous bytes of each of its two rows per chunk, as in the packed layout).
// Activations go global -> LDS by LDS DMA (16 bytes per lane, 1 KiB = 4 staged
// rows per wave load; the lane's global column is chosen so that slot s of
// staged row r holds column piece s ^ (r % 16)), so they take no registers.
// Dequantisation as fp8x8_dequant (exact decode, one fp32 multiply by the
// 128 x 128 block scale, one rounding to bf16).
constexpr int kF8BM = 96;                                           // activation rows per tile
constexpr int kF8MB = kF8BM / 32;                                   // MFMA row blocks per tile
constexpr int kF8Waves = 8;                                         // waves per workgroup
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8NB = kF8Waves / 2;                                 // N blocks per tile
constexpr int kF8Grid = 256;                                        // 1 resident workgroup x 256 CUs
constexpr int kF8PartFloats = kF8Waves * 2 * kF8MB * 16 * kWave;   // one workgroup's accumulators (192 KiB)
static_assert(kF8Threads <= kMaxGemmThreads, "schedule scratch holds one entry per thread");

__device__ __forceinline__ float* f8_slot(float* parts, int b, int slot) {
  return parts + (size_t(b) * 2 + slot) * kF8PartFloats;
}
// [wave][a][block][quad q][lane][4 floats]: 1 KiB contiguous per wave access
__device__ __forceinline__ int f8_part_idx(int wv, int a, int b, int q, int lane) {
  return ((((wv * 2 + a) * kF8MB + b) * 4 + q) * kWave + lane) * 4;
}

// Tiles (of four N blocks) tl.nt .. tl.nt + n - 1 of one group and row tile,
// iterations [it_begin, it_end) of the run (as bf_run: with one row tile the
// group's next tiles read the same activation rows, so the loads run ahead
// across tile boundaries).
template <int KIND, bool PACKED, int NB, bool STREAM>
__device__ __forceinline__ void f8_run(const GemmArgs& p, const Tile& tl, int n, const Sched& sh,
                                       uint16_t* __restrict__ x0, uint16_t* __restrict__ x1,
                                       uint16_t* __restrict__ x2, int it_begin, int it_end,
                                       float* __restrict__ part_first, float* __restrict__ part_last) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar
  const int wq = wv & 3;   // the wave's 32 rows of each N block
  const int wg = wv >> 2;  // the wave's pair of N blocks in the tile
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nchunks = __builtin_amdgcn_readfirstlane(p.K / kKC);
  it_begin = __builtin_amdgcn_readfirstlane(it_begin);
  it_end = __builtin_amdgcn_readfirstlane(it_end);
  n = __builtin_amdgcn_readfirstlane(n);
  const int last = it_end - 1;
  // N block of sub-block a of the run's tile k (past the group's last block a
  // sub-block repeats it; its results are discarded)
  // (operands in scalar registers, so the arithmetic on them stays scalar)
  const int nt0 = __builtin_amdgcn_readfirstlane(kF8NB * tl.nt + 2 * wg);
  const int nt_max = __builtin_amdgcn_readfirstlane(p.n_tiles_n - 1);
  auto ntof = [&](int k, int a) { return min(nt0 + kF8NB * k + a, nt_max); };

  // weights: uniform base (the expert's block) + the lane's loop-invariant byte
  // offset (its row in N block 0; an expert's weights span less than 4 GiB)
  const uint8_t* W = static_cast<const uint8_t*>(pick(tl.shared, p.sh_w, p.w));
  int wrow0;  // this lane's weight row in N block 0
  if (KIND == kUp) {
    const int j = 16 * wq + (lr & 15);
    wrow0 = lr < 16 ? j : p.n_out + j;
  } else {
    wrow0 = 32 * wq + lr;
  }
  // Weights and scales come by buffer loads (see buf_rsrc) from a resource at
  // the expert's base, with a scalar offset per (N block, chunk) and a
  // loop-invariant lane offset. (The activations go to LDS by global_load_lds
  // (lds_dma16_untracked): the buffer form of the LDS copy is not used, its
  // LDS addressing on this chip - scalar offset, destinations above 64 KiB -
  // not being established.)
  __amdgpu_buffer_rsrc_t rw;
  uint32_t woff;
  if constexpr (PACKED) {
    rw = buf_rsrc(W + size_t(tl.we) * p.n_tiles_n * nchunks * 4 * 4 * kWave * 16);
    woff = uint32_t(wq * 4 * kWave + lane) * 16u;
  } else {
    rw = buf_rsrc(W + size_t(tl.we) * p.n_w_rows * p.K);
    woff = uint32_t(wrow0 * p.K + 64 * lh);
  }
  // iteration I = k * nchunks + C, sub-block a: scalar offset of its piece 0
  // (piece j lies j KiB (packed) or 16 j bytes (row-major) further)
  auto wsoff = [&](int k, int C, int a) -> int {
    const int nt = ntof(k, a);
    if constexpr (PACKED) return (nt * nchunks + C) * 4 * 4 * kWave * 16;
    else return nt * (KIND == kUp ? 64 : 128) * p.K + C * kKC;
  };
  auto wpiece = [&](int k, int C, int a, int j) -> uint4 {
    constexpr int aux = STREAM ? 2 : 0;  // non-temporal: the weights are read once
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
        rw, woff, __builtin_amdgcn_readfirstlane(wsoff(k, C, a) + (PACKED ? j * kWave * 16 : j * 16)), aux);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // block scales: 128-row blocks; up: gate rows of N block nt lie in block
  // nt / 2, its up rows in block I / 128 + nt / 2; down: block nt
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(pick(tl.shared, p.sh_s, p.s) + size_t(tl.we) * (p.n_w_rows / 128) * nchunks);
  const uint32_t s_lane = KIND == kUp && lr >= 16 ? uint32_t(p.n_out / 128) * nchunks * 4u : 0u;
  auto scale = [&](int k, int C, int a) {
    const int nt = ntof(k, a);
    const int so = ((KIND == kUp ? nt >> 1 : nt) * nchunks + C) * 4;
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, s_lane, __builtin_amdgcn_readfirstlane(so), 0));
  };

  // activations: load q of this wave stages tile rows 4 (8 q + wv) .. + 3
  constexpr int XL = NB * 8 / kF8Waves;  // 1 KiB loads per wave per chunk
  const uint16_t* A = static_cast<const uint16_t*>(pick(tl.shared, p.sh_a, p.a));
  const bool ablk = pick(tl.shared, p.sh_a_blk, p.a_blk);
  const size_t xstep = ablk ? size_t(4) * 512 : size_t(kKC);  // elements from one chunk of a row to the next
  // per-lane byte offsets from the tile's first row (a tile's rows lie in one
  // expert's region, which the host keeps below 2^31 elements); gathered rows
  // from a's start (the host keeps a below 2^32 bytes)
  const bool gat = p.a_rows != nullptr && !tl.shared;
  const int* amap = gat ? sh.arow : sh.rowmap;
  const int phys0 = amap[0];
  const size_t xbase = gat ? 0 : ablk ? blk_row_base(phys0, p.K) : size_t(phys0) * p.K;
  const gptr<char> xb = uniform_ptr(reinterpret_cast<const char*>(A + xbase));
  uint32_t xoff[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int r = 4 * (kF8Waves * q + wv) + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);  // column piece this lane's LDS slot holds
    const int phys = r < NB * 32 ? amap[r] : -1;
    const int pr = phys >= 0 ? phys : phys0;  // rows past the tile feed only discarded columns
    xoff[q] = uint32_t((ablk ? blk_row_base(pr, p.K) + size_t(c >> 2) * 512 + (c & 3) * 8 : size_t(pr) * p.K + c * 8) -
                       xbase) * 2u;
  }

  f32x16_t acc[2][NB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));

  // Ring. Iteration I of the run (counted from it_begin) takes activation
  // buffer and scale pair (I - it_begin) % 3 and weight set (I - it_begin) % 2.
  // At the top of iteration I (after the barrier: every wave has left I - 1,
  // the last reader of that buffer) go out the activation DMA and the scales
  // of I + 2; piece j of the weights of I + 2 replaces piece j of I's set as
  // soon as the dequantisation of I has read it for the last time (steps 0,
  // 2, 4, 6). Every operand is so requested about two iterations before its
  // use, with the registers of two. A wave's vector-memory ops per iteration,
  // in issue order: XL activation DMAs, 2 scale loads, 2 weight loads at each
  // of steps 0, 2, 4 and 6 (XL + 10); they retire in order (epilogue stores
  // in between only make a count wait longer), so
  //  - at the top of I, the activations, scales and piece 0 of I are followed
  //    by pieces 1-3 of I (6 ops) and all of I + 1: vmcnt(XL + 16);
  //  - piece j = 1, 2, 3 of I, first read in step 2j - 1, is followed by the
  //    2 (3 - j) later pieces of I, all of I + 1 and, of I + 2, the top loads
  //    and pieces 0 .. j - 1: vmcnt(2 XL + 18) in each case.
  // (Past the run's end the loads repeat its last iteration, so the counts
  // hold.) Inside an iteration, one 16-deep step at a time (fenced, so the
  // compiler cannot hoist a whole iteration of fragment reads): step j reads
  // its activation fragments, dequantises the weights of step j + 1 and
  // issues its MFMAs with the fragments dequantised before.
  // LDS fragment of row block b in step j: row 32 b + lr, 16-byte column
  // (8 lh + j) ^ (lr % 16) = (8 lh ^ (lr & 8)) + (j ^ (lr & 7)); the lane's
  // part is rebuilt from an opaque copy each iteration, so the compiler does
  // not hold the eight step addresses in registers for the whole loop
  const int fr_base = lr * kKC + ((8 * lh) ^ (lr & 8)) * 8;
  const int fr_x = lr & 7;
  uint4 w0[2][4], w1[2][4];   // weight sets [sub-block][piece]
  float s0[2], s1[2], s2[2];  // block scales per sub-block
  bf16x8_t fa[2];             // weight fragments of the current step
  // (tile k of the run, chunk c) of the iteration being computed and of the
  // one being loaded, kept as counters (an integer division per iteration
  // would be done by the vector ALU)
  int k_cur = __builtin_amdgcn_readfirstlane(it_begin / nchunks);
  int c_cur = __builtin_amdgcn_readfirstlane(it_begin - k_cur * nchunks);
  int i_ld = it_begin, k_ld = k_cur, c_ld = c_cur;
  // (readfirstlane: the counters are uniform; it keeps the compiler from
  // moving them and the address arithmetic on them to vector registers)
  auto adv_ld = [&]() __attribute__((always_inline)) {  // to the next iteration, but not past the last
    if (i_ld < last) {
      ++i_ld;
      if (++c_ld == nchunks) {
        c_ld = 0;
        ++k_ld;
      }
    }
    i_ld = __builtin_amdgcn_readfirstlane(i_ld);
    c_ld = __builtin_amdgcn_readfirstlane(c_ld);
    k_ld = __builtin_amdgcn_readfirstlane(k_ld);
  };
#define MOE_F8_TOP(XBUF_, SR_)                                                                              \
  {                                                                                                         \
    const int k_ = k_ld, c_ = c_ld;                                                                         \
    const gptr<char> xc_ = xb + uint64_t(c_) * xstep * 2; /* the chunk's base: scalar */                   \
    _Pragma("unroll") for (int q = 0; q < XL; ++q)                                                          \
      lds_dma16_untracked(xc_, xoff[q], (XBUF_) + (kF8Waves * q + wv) * 512);                               \
    _Pragma("unroll") for (int a = 0; a < 2; ++a) SR_[a] = scale(k_, c_, a);                                \
  }
#define MOE_F8_PIECE(WR_, J_)                                                                               \
  _Pragma("unroll") for (int a = 0; a < 2; ++a) WR_[a][J_] = wpiece(k_ld, c_ld, a, J_);
#define MOE_F8_DEQ(DST_, WR_, J_, SR_)                                                                      \
  _Pragma("unroll") for (int a = 0; a < 2; ++a) DST_[a] =                                                   \
      ((J_) & 1) ? fp8x8_dequant(WR_[a][(J_) >> 1].z, WR_[a][(J_) >> 1].w, SR_[a])                          \
                 : fp8x8_dequant(WR_[a][(J_) >> 1].x, WR_[a][(J_) >> 1].y, SR_[a]);
  // the 8 steps of an iteration (activations XBUF_, weights WR_, scales SR_);
  // refills WR_ with the pieces of the iteration being loaded
#define MOE_F8_STEPS(XBUF_, WR_, SR_)                                                                       \
  int fx_ = fr_x;                                                                                           \
  asm volatile("" : "+v"(fx_));                                                                             \
  _Pragma("unroll") for (int j = 0; j < 8; ++j) {                                                           \
    const int fo_ = fr_base + ((j ^ fx_) * 8); /* 16-byte column: k = 64 lh + 8 j */                        \
    bf16x8_t fb_[NB];                                                                                       \
    _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                          \
      fb_[b] = *reinterpret_cast<const bf16x8_t*>((XBUF_) + b * 32 * kKC + fo_);                             \
    bf16x8_t na_[2];                                                                                        \
    if (j < 7) {                                                                                            \
      if (j & 1) {                                                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                                  \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * XL + 18));                                                \
        __builtin_amdgcn_sched_barrier(0);                                                                  \
      }                                                                                                     \
      MOE_F8_DEQ(na_, WR_, j + 1, SR_)                                                                      \
      if (!(j & 1)) { MOE_F8_PIECE(WR_, j >> 1) }                                                           \
    }                                                                                                       \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                        \
      acc[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb_[b], acc[0][b], 0, 0, 0);               \
      acc[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb_[b], acc[1][b], 0, 0, 0);               \
    }                                                                                                       \
    if (j < 7) {                                                                                            \
      fa[0] = na_[0];                                                                                       \
      fa[1] = na_[1];                                                                                       \
    }                                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
  }
  // after iteration I_: if it ends its tile, the tile's epilogue (or partial
  // sums) and fresh accumulators
#define MOE_F8_FINISH(I_)                                                                                   \
  {                                                                                                         \
    const int k_ = k_cur;                                                                                   \
    if (c_cur == nchunks - 1 || (I_) == last) { /* uniform */                                               \
      float* part_ = k_ == 0 ? part_first : (k_ == n - 1 ? part_last : nullptr);                            \
      if (part_ == nullptr) {                                                                               \
        _Pragma("unroll") for (int a = 0; a < 2; ++a) {                                                     \
          Tile ta_ = tl;                                                                                    \
          ta_.nt = kF8NB * (tl.nt + k_) + 2 * wg + a;                                                       \
          if (ta_.nt < p.n_tiles_n) ffn_epilogue<KIND, NB>(acc[a], ta_, NB, sh, out, p.n_out, wq, lr, lh, p.out_blk); \
        }                                                                                                   \
      } else {                                                                                              \
        _Pragma("unroll") for (int a = 0; a < 2; ++a)                                                       \
          _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                    \
            _Pragma("unroll") for (int v = 0; v < 16; v += 4)                                               \
              *reinterpret_cast<float4*>(part_ + f8_part_idx(wv, a, b, v / 4, lane)) =                      \
                  make_float4(acc[a][b][v], acc[a][b][v + 1], acc[a][b][v + 2], acc[a][b][v + 3]);          \
      }                                                                                                     \
      _Pragma("unroll") for (int a = 0; a < 2; ++a)                                                         \
        _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                      \
          _Pragma("unroll") for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;                                \
    }                                                                                                       \
    if (++c_cur == nchunks) {                                                                               \
      c_cur = 0;                                                                                            \
      ++k_cur;                                                                                              \
    }                                                                                                       \
    c_cur = __builtin_amdgcn_readfirstlane(c_cur);                                                          \
    k_cur = __builtin_amdgcn_readfirstlane(k_cur);                                                          \
  }
  // iteration I_ in (XBUF_, WR_, SR_); the activations and scales of I_ + 2 go to (XN_, SN_)
#define MOE_F8_ITER(I_, XBUF_, WR_, SR_, XN_, SN_)                                                          \
  {                                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(XL + 16));                                                  \
    __builtin_amdgcn_s_barrier();                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    adv_ld(); /* to min(I_ + 2, last): past the end a harmless repeat */                                    \
    MOE_F8_TOP(XN_, SN_)                                                                                    \
    MOE_F8_DEQ(fa, WR_, 0, SR_)                                                                             \
    MOE_F8_STEPS(XBUF_, WR_, SR_)                                                                           \
    MOE_F8_FINISH(I_)                                                                                       \
  }

  MOE_F8_TOP(x0, s0)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    MOE_F8_PIECE(w0, j)
  }
  adv_ld();
  MOE_F8_TOP(x1, s1)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    MOE_F8_PIECE(w1, j)
  }
  // six iterations per trip (the ring periods are 3 and 2), then up to five
  // in a tail with the same slots. (No exit in the middle of a trip: the
  // accumulators would need a second copy at the exit, and the wait counts of
  // the loop head would have to cover the shorter trips.)
  int it = it_begin;
  for (; it + 6 <= it_end; it += 6) {
    MOE_F8_ITER(it, x0, w0, s0, x2, s2)
    MOE_F8_ITER(it + 1, x1, w1, s1, x0, s0)
    MOE_F8_ITER(it + 2, x2, w0, s2, x1, s1)
    MOE_F8_ITER(it + 3, x0, w1, s0, x2, s2)
    MOE_F8_ITER(it + 4, x1, w0, s1, x0, s0)
    MOE_F8_ITER(it + 5, x2, w1, s2, x1, s1)
  }
  if (it < it_end) {
    MOE_F8_ITER(it, x0, w0, s0, x2, s2)
    if (it + 1 < it_end) {
      MOE_F8_ITER(it + 1, x1, w1, s1, x0, s0)
      if (it + 2 < it_end) {
        MOE_F8_ITER(it + 2, x2, w0, s2, x1, s1)
        if (it + 3 < it_end) {
          MOE_F8_ITER(it + 3, x0, w1, s0, x2, s2)
          if (it + 4 < it_end) MOE_F8_ITER(it + 4, x1, w0, s1, x0, s0)
        }
      }
    }
  }
#undef MOE_F8_ITER
#undef MOE_F8_FINISH
#undef MOE_F8_STEPS
#undef MOE_F8_DEQ
#undef MOE_F8_PIECE
#undef MOE_F8_TOP
  // no load may still be writing LDS when the next run reuses the buffers
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
}

// Stream-K over (tile, chunk) iterations as ffn_bf16_kernel, with tiles of 96
// rows x four N blocks over at most kF8Grid ranges, streamed in runs as there.
template <int KIND, bool PACKED>
__global__ __launch_bounds__(kF8Threads, 1) void ffn_fp8_kernel(GemmArgs p, float* __restrict__ parts) {
  __shared__ Sched sh;
  __shared__ __attribute__((aligned(1024))) uint16_t x0[kF8BM * kKC], x1[kF8BM * kKC], x2[kF8BM * kKC];
  const int ntn4 = (p.n_tiles_n + kF8NB - 1) / kF8NB;
  const int n_tiles = build_schedule<kF8Threads>(p, kF8BM, ntn4, false, sh);
  const int nchunks = p.K / kKC;
  const int64_t total = int64_t(n_tiles) * nchunks;
  const int G = sk_grid(total, kF8Grid);
  if (int(blockIdx.x) >= G) return;  // uniform
  const int rng = int(blockIdx.x % kXcds) * (G / kXcds) + int(blockIdx.x / kXcds);
  const int64_t i0 = sk_start(rng, total, G), i1 = sk_start(rng + 1, total, G);
  if (i0 >= i1) return;  // uniform
  const int t_first = int(i0 / nchunks), t_last = int((i1 - 1) / nchunks);
  for (int t = t_first; t <= t_last;) {
    const Tile tl = decode_tile(p, kF8BM, ntn4, sh, t);
    build_rowmap<kF8Threads>(p, tl, kF8BM, sh, true);
    const int n = tl.mtiles == 1 ? min(t_last - t + 1, ntn4 - tl.nt) : 1;
    const int64_t t0 = int64_t(t) * nchunks;
    const int it_begin = int(max<int64_t>(i0 - t0, 0));
    const int it_end = int(min<int64_t>(i1 - t0, int64_t(n) * nchunks));
    const bool split_first = it_begin > 0 || (n == 1 && it_end < nchunks);
    const bool split_last = it_end < n * nchunks;
    float* part_first = split_first ? f8_slot(parts, rng, t == t_first ? 0 : 1) : nullptr;
    float* part_last = n == 1 ? part_first : (split_last ? f8_slot(parts, rng, 1) : nullptr);
    auto run = [&](auto stream_tag) __attribute__((always_inline)) {
      constexpr bool ST = decltype(stream_tag)::value;
      switch ((tl.nrows + 31) / 32) {
        case 1: f8_run<KIND, PACKED, 1, ST>(p, tl, n, sh, x0, x1, x2, it_begin, it_end, part_first, part_last); break;
        case 2: f8_run<KIND, PACKED, 2, ST>(p, tl, n, sh, x0, x1, x2, it_begin, it_end, part_first, part_last); break;
        default: f8_run<KIND, PACKED, 3, ST>(p, tl, n, sh, x0, x1, x2, it_begin, it_end, part_first, part_last); break;
      }
    };
    if (tl.mtiles == 1) run(std::true_type{});
    else run(std::false_type{});
    __syncthreads();  // rowmap is rewritten by the next run
    t += n;
  }
}

// Finishes the fp8 tiles cut by a range boundary (as ffn_fixup_kernel); block
// (j, m * kF8MB + b) takes the tile's N block m, 32-row block b, with one wave
// per 32 rows of the block (the partials of the main kernel's waves m / 2 * 4
// .. + 3, sub-block m % 2).
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_fp8_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int ntn4 = (p.n_tiles_n + kF8NB - 1) / kF8NB;
  const int n_tiles = build_schedule(p, kF8BM, ntn4, false, sh);
  const int nchunks = p.K / kKC;
  const int64_t total = int64_t(n_tiles) * nchunks;
  const int j = blockIdx.x, m = blockIdx.y / kF8MB, b = blockIdx.y % kF8MB;
  const int G = sk_grid(total, kF8Grid);
  if (j + 1 >= G) return;  // uniform: boundaries lie between ranges 0 .. G-1
  const int64_t ib = sk_start(j + 1, total, G);
  if (ib <= 0 || ib >= total || ib % nchunks == 0) return;  // not inside a tile
  const int t = int(ib / nchunks);
  if (j > 0 && sk_start(j, total, G) > int64_t(t) * nchunks) return;  // an earlier boundary owns this tile
  Tile tl = decode_tile(p, kF8BM, ntn4, sh, t);
  if (b * 32 >= tl.nrows || kF8NB * tl.nt + m >= p.n_tiles_n) return;  // uniform: no rows / no such N block
  build_rowmap(p, tl, kF8BM, sh);
  const int b_lo = sk_owner(int64_t(t) * nchunks, total, G);
  const int b_hi = sk_owner(int64_t(t + 1) * nchunks - 1, total, G);
  f32x16_t acc[1];
  sum_partials(
      acc, b_lo, b_hi,
      [&](int w) -> const float* {
        const int64_t s0 = sk_start(w, total, G), s1 = sk_start(w + 1, total, G);
        return s0 < s1 ? f8_slot(const_cast<float*>(parts), w, int(s0 / nchunks) == t ? 0 : 1) : nullptr;
      },
      [&](int, int q) { return f8_part_idx(m / 2 * 4 + wv, m % 2, b, q, lane); });
  tl.nt = kF8NB * tl.nt + m;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  ffn_epilogue_block<KIND>(acc[0], tl, b, sh, out, p.n_out, wv, lr, lh, p.out_blk);
}

// ------------------------------------------------------------------ weight packing
// Packed layout: for expert g, N block nt (64 h columns = 128 rows of W13, or
// 128 rows of W2) and 128-deep K chunk c, the 32 rows x 128 k of each of the 4
// waves, in the order the lanes of the decode kernels load them:
// [g][nt][c][wave][load i][lane][16 bytes]. One load instruction of a wave then
// reads 1 KiB of contiguous memory and a workgroup streams one sequential
// region, instead of 128 rows in 256-byte pieces. It is a permutation of the
// row-major bytes (same size); one thread moves one 16-byte piece.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ src, uint4* __restrict__ dst,
                                                           int64_t n_pieces, int kind, int fp8, int n_w_rows, int K,
                                                           int n_out, int n_tiles_n) {
  const int WV = fp8 ? 4 : 8;
  const int eb = fp8 ? 1 : 2;
  const int nchunks = K / kKC;
  for (int64_t d = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; d < n_pieces;
       d += int64_t(gridDim.x) * blockDim.x) {
    const int l = int(d % kWave);
    int64_t q = d / kWave;
    const int i = int(q % WV);
    q /= WV;
    const int w = int(q % 4);
    q /= 4;
    const int c = int(q % nchunks);
    q /= nchunks;
    const int nt = int(q % n_tiles_n);
    const int64_t g = q / n_tiles_n;
    const int r = l & 31, h = l >> 5;
    int row;
    if (kind == kUp) {
      const int j = nt * 64 + 16 * w + (r & 15);
      row = r < 16 ? j : n_out + j;
    } else {
      row = nt * 128 + 32 * w + r;
    }
    const int k = fp8 ? c * kKC + 64 * h + 16 * i : c * kKC + 64 * (i >> 2) + 32 * h + 8 * (i & 3);
    dst[d] = *reinterpret_cast<const uint4*>(src + ((g * n_w_rows + row) * int64_t(K) + k) * eb);
  }
}

// ------------------------------------------------------------------ fp32 SIMT kernel
constexpr int kFBM = 32;  // rows per tile
constexpr int kFBN = 32;  // output columns per tile
constexpr int kFKC = 32;  // reduction chunk

template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_f32_kernel(GemmArgs p) {
  __shared__ Sched sh;
  __shared__ float xs[kFBM][kFKC + 1];
  __shared__ float ws[2 * kFBN][kFKC + 1];
  const int tid = threadIdx.x;
  const int n_tiles = build_schedule(p, kFBM, p.n_tiles_n, false, sh);
  const int nwr = KIND == kUp ? 2 * kFBN : kFBN;  // weight rows staged per tile
  const int row = tid / 8;                         // 0..31
  const int cg = (tid % 8) * 4;                    // 4 output columns

  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const Tile tl = decode_tile(p, kFBM, p.n_tiles_n, sh, t);
    build_rowmap(p, tl, kFBM, sh);
    const float* A = static_cast<const float*>(pick(tl.shared, p.sh_a, p.a));
    const float* W = static_cast<const float*>(pick(tl.shared, p.sh_w, p.w));
    float* out = static_cast<float*>(pick(tl.shared, p.sh_out, p.out));
    float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.K; k0 += kFKC) {
      for (int i = tid; i < kFBM * kFKC; i += kGemmThreads) {
        const int r = i / kFKC, k = i % kFKC;
        const int phys = sh.rowmap[r];
        xs[r][k] = phys >= 0 ? A[size_t(phys) * p.K + k0 + k] : 0.f;
      }
      for (int i = tid; i < nwr * kFKC; i += kGemmThreads) {
        const int r = i / kFKC, k = i % kFKC;
        int wr;
        if (KIND == kUp) wr = r < kFBN ? tl.nt * kFBN + r : p.n_out + tl.nt * kFBN + (r - kFBN);
        else wr = tl.nt * kFBN + r;
        ws[r][k] = W[(size_t(tl.we) * p.n_w_rows + wr) * p.K + k0 + k];
      }
      __syncthreads();
#pragma unroll 4
      for (int k = 0; k < kFKC; ++k) {
        const float xv = xs[row][k];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          g[c] = fmaf(xv, ws[cg + c][k], g[c]);
          if (KIND == kUp) u[c] = fmaf(xv, ws[kFBN + cg + c][k], u[c]);
        }
      }
      __syncthreads();
    }
    const int phys = sh.rowmap[row];
    if (phys >= 0) {
      float* orow = out + size_t(phys) * p.n_out + tl.nt * kFBN + cg;
#pragma unroll
      for (int c = 0; c < 4; ++c) orow[c] = KIND == kUp ? silu_f(g[c]) * u[c] : g[c];
    }
    __syncthreads();
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

static bool ggemm_desc_ok(const moe_ggemm_desc_t* d) {
  if (!d) return false;
  if (d->n_groups < 0 || d->hidden < 1 || d->inter < 1 || d->rows < 0) return false;
  if (d->layout != MOE_LAYOUT_COMPACT && d->layout != MOE_LAYOUT_PADDED) return false;
  if (d->stage != MOE_GG_FULL && d->stage != MOE_GG_UP && d->stage != MOE_GG_DOWN) return false;
  if (d->layout == MOE_LAYOUT_PADDED) {
    if (d->n_src < 1 || d->capacity < 0) return false;
    if (int64_t(d->n_groups) * d->n_src * d->capacity > d->rows) return false;
  }
  if (d->shared && d->shared->rows < 0) return false;
  if (d->w_format != MOE_W_ROWMAJOR && d->w_format != MOE_W_PACKED) return false;
  if (d->policy != MOE_GEMM_AUTO && d->policy != MOE_GEMM_WIDE && d->policy != MOE_GEMM_STREAM_K) return false;
  if (d->a_layout != MOE_ACT_ROWS && d->a_layout != MOE_ACT_BLOCKED16) return false;
  if (d->a_rows && d->a_nrows < 1) return false;
  return true;
}

static bool ggemm_desc_supported(const moe_ggemm_desc_t* d) {
  const bool f32 = d->act_dt == MOE_F32 && d->w_dt == MOE_F32;
  const bool bf16 = d->act_dt == MOE_BF16 && (d->w_dt == MOE_BF16 || d->w_dt == MOE_FP8_E4M3);
  if (!f32 && !bf16) return false;
  if (d->hidden % 128 || d->inter % 128) return false;
  if (d->n_groups > kMaxGroups) return false;
  if (d->layout == MOE_LAYOUT_PADDED && d->n_src > kGemmMaxSrc) return false;
  if (d->rows >= (int64_t(1) << 31)) return false;
  if (d->shared && d->shared->rows >= (1 << 30)) return false;
  if (f32 && d->w_format == MOE_W_PACKED) return false;
  if (f32 && d->a_layout != MOE_ACT_ROWS) return false;
  // gathering: row-major bf16 rows, 32-bit byte offsets (decode-shaped kernels)
  if (d->a_rows && (f32 || d->a_layout != MOE_ACT_ROWS ||
                    d->a_nrows > (int64_t(1) << 32) / (int64_t(d->hidden) * 2)))
    return false;
  return true;
}

// h [rows, I]: fp32 row-major, or bf16 in the 16-row blocked layout (rows
// rounded up to 16)
static size_t h_bytes(const moe_ggemm_desc_t* d, int64_t rows) {
  const size_t el = d->act_dt == MOE_F32 ? 4 : 2;
  if (d->act_dt != MOE_F32) rows = (rows + 15) / 16 * 16;
  return align_up(size_t(rows) * size_t(d->inter) * el, 256);
}

static size_t parts_bytes(const moe_ggemm_desc_t* d) {
  // shared by the wide and the stream-K kernels, which run one after the other
  const size_t sk = d->w_dt == MOE_FP8_E4M3 ? size_t(2) * kF8Grid * kF8PartFloats : size_t(2) * kBfGrid * kPartFloats;
  const size_t wide = size_t(kWideGrid) * kWidePart;
  return d->act_dt == MOE_F32 ? 0 : std::max(sk, wide) * sizeof(float);
}

MOE_API size_t moe_grouped_gemm_workspace(const moe_ggemm_desc_t* d) {
  if (!ggemm_desc_ok(d)) return 0;
  const int64_t sh_rows = d->shared ? d->shared->rows : 0;
  return h_bytes(d, d->rows) + h_bytes(d, sh_rows) + parts_bytes(d) + 256;
}

namespace moe {
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
  if (dev < 64) cached[dev] = cu;
  return cu;
}
}  // namespace moe

// sk: launch the stream-K kernel (false only when the wide kernel takes every group)
static moe_status_t launch_stage(const GemmArgs& p, bool f32, bool fp8, int kind, bool sk, float* parts,
                                 hipStream_t stream) {
  const dim3 block(kGemmThreads);
  if (f32) {
    const int64_t upper = int64_t(p.n_tiles_n) * ((p.rows + kFBM - 1) / kFBM + p.G + (p.sh_rows + kFBM - 1) / kFBM + 1);
    const int64_t resident = int64_t(device_cu_count()) * 4;
    const dim3 grid(unsigned(upper < resident ? upper : resident));
    if (kind == kUp) hipLaunchKernelGGL(ffn_f32_kernel<kUp>, grid, block, 0, stream, p);
    else hipLaunchKernelGGL(ffn_f32_kernel<kDown>, grid, block, 0, stream, p);
    return launch_status();
  }
  if (p.wide_min != kNoWide) {
    const dim3 wgrid(kWideGrid);
#define MOE_WIDE(K, P) hipLaunchKernelGGL((ffn_wide_kernel<K, P>), wgrid, block, 0, stream, p, parts)
    if (kind == kUp) { if (p.packed) MOE_WIDE(kUp, true); else MOE_WIDE(kUp, false); }
    else { if (p.packed) MOE_WIDE(kDown, true); else MOE_WIDE(kDown, false); }
#undef MOE_WIDE
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    // the partials are finished before the stream-K kernel reuses the buffer
    const dim3 wfix(kWideGrid, 8);
    if (kind == kUp) hipLaunchKernelGGL((ffn_wide_fixup_kernel<kUp>), wfix, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_wide_fixup_kernel<kDown>), wfix, block, 0, stream, p, parts);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    if (!sk) return launch_status();
  }
  if (fp8) {
    const dim3 f8_grid(kF8Grid), f8_block(kF8Threads);
#define MOE_F8(K, P) hipLaunchKernelGGL((ffn_fp8_kernel<K, P>), f8_grid, f8_block, 0, stream, p, parts)
    if (kind == kUp) { if (p.packed) MOE_F8(kUp, true); else MOE_F8(kUp, false); }
    else { if (p.packed) MOE_F8(kDown, true); else MOE_F8(kDown, false); }
#undef MOE_F8
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    const dim3 fix_grid(kF8Grid - 1, kF8NB * kF8MB);
    if (kind == kUp) hipLaunchKernelGGL((ffn_fp8_fixup_kernel<kUp>), fix_grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_fp8_fixup_kernel<kDown>), fix_grid, block, 0, stream, p, parts);
    return launch_status();
  }
  const dim3 bf_grid(kBfGrid), bf_block(kBfThreads);
#define MOE_FFN(K, P) hipLaunchKernelGGL((ffn_bf16_kernel<K, P>), bf_grid, bf_block, 0, stream, p, parts)
  if (kind == kUp) { if (p.packed) MOE_FFN(kUp, true); else MOE_FFN(kUp, false); }
  else { if (p.packed) MOE_FFN(kDown, true); else MOE_FFN(kDown, false); }
#undef MOE_FFN
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 fix_grid(kBfGrid - 1, kBfNB * kBfMB);
  if (kind == kUp) hipLaunchKernelGGL((ffn_fixup_kernel<kUp>), fix_grid, block, 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_fixup_kernel<kDown>), fix_grid, block, 0, stream, p, parts);
  return launch_status();
}

MOE_API moe_status_t moe_grouped_gemm(const moe_ggemm_desc_t* d, const void* a, const int32_t* counts,
                                      const int32_t* group_off, const void* w13, const void* w2, const float* s13,
                                      const float* s2, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ggemm_desc_ok(d)) return MOE_ERR_INVALID_ARG;
  if (!ggemm_desc_supported(d)) return MOE_ERR_UNSUPPORTED;
  const moe_shared_expert_t* se = (d->shared && d->shared->rows > 0) ? d->shared : nullptr;
  const bool routed = d->n_groups > 0 && d->rows > 0;
  if (!routed && !se) return MOE_OK;
  const bool f32 = d->act_dt == MOE_F32;
  const bool fp8 = d->w_dt == MOE_FP8_E4M3;
  const bool up = d->stage != MOE_GG_DOWN, down = d->stage != MOE_GG_UP;
  if (routed) {
    if (d->layout == MOE_LAYOUT_COMPACT && !group_off) return MOE_ERR_INVALID_ARG;
    if (d->layout == MOE_LAYOUT_PADDED && !counts) return MOE_ERR_INVALID_ARG;
    if (up && (!a || !w13 || !aligned16(a) || !aligned16(w13))) return MOE_ERR_INVALID_ARG;
    if (down && (!y || !w2 || !aligned16(y) || !aligned16(w2))) return MOE_ERR_INVALID_ARG;
    if (fp8 && ((up && !s13) || (down && !s2))) return MOE_ERR_INVALID_ARG;
  }
  if (se) {
    if (up && (!se->a || !se->w13 || !aligned16(se->a) || !aligned16(se->w13))) return MOE_ERR_INVALID_ARG;
    if (down && (!se->y || !se->w2 || !aligned16(se->y) || !aligned16(se->w2))) return MOE_ERR_INVALID_ARG;
    if (fp8 && ((up && !se->s13) || (down && !se->s2))) return MOE_ERR_INVALID_ARG;
  }
  if (!ws || !aligned16(ws) || ws_bytes < moe_grouped_gemm_workspace(d)) return MOE_ERR_WORKSPACE;
  // the decode kernels address a tile's activation rows relative to its first
  // row: one expert's padded region must span fewer than 2^31 elements
  if (!f32 && d->layout == MOE_LAYOUT_PADDED &&
      (int64_t(d->n_src) * d->capacity + 16) * std::max(d->hidden, d->inter) >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;

  void* h = ws;
  void* sh_h = static_cast<char*>(ws) + h_bytes(d, d->rows);
  float* parts = reinterpret_cast<float*>(static_cast<char*>(sh_h) + h_bytes(d, d->shared ? d->shared->rows : 0));
  GemmArgs p;
  p.rows = routed ? d->rows : 0;
  p.counts = counts;
  p.group_off = group_off;
  p.G = routed ? d->n_groups : 0;
  p.S = d->layout == MOE_LAYOUT_PADDED ? d->n_src : 1;
  p.C = d->layout == MOE_LAYOUT_PADDED ? d->capacity : 0;
  p.layout = d->layout;
  p.sh_rows = se ? se->rows : 0;
  p.packed = d->w_format == MOE_W_PACKED;
  // the wide-tile kernel: bf16 weights, 256-row output blocks of W2 and 128-column blocks of h
  const bool wide_ok = !f32 && !fp8 && d->hidden % 256 == 0 && d->inter % 128 == 0 &&
                       d->policy != MOE_GEMM_STREAM_K;
  const bool force = d->policy == MOE_GEMM_WIDE;
  p.wide_min = wide_ok ? (force ? 1 : kWideMinRows) : kNoWide;
  const bool sk = !(wide_ok && force);  // forced wide leaves the stream-K kernel nothing
  // h (internal) in the 16-row blocked layout where the wide kernel may run
  // (its loads take 16 rows x 32 columns); row-major for the decode kernels,
  // whose loads take 4 rows x 128 columns
  const bool h_blk = wide_ok;
  p.wide_min_tiles = force ? 0 : kWideMinTiles;
  p.sh_a_blk = 0;
  p.a_rows = nullptr;
  p.a_nrows = 0;
  moe_status_t st = MOE_OK;
  if (up) {
    p.a = a;
    p.a_rows = d->a_rows;
    p.a_nrows = d->a_rows ? int(d->a_nrows) : 0;
    p.w = w13;
    p.s = s13;
    p.out = h;
    p.sh_a = se ? se->a : nullptr;
    p.sh_w = se ? se->w13 : nullptr;
    p.sh_s = se ? se->s13 : nullptr;
    p.sh_out = sh_h;
    p.n_w_rows = 2 * d->inter;
    p.K = d->hidden;
    p.n_out = d->inter;
    p.n_tiles_n = f32 ? d->inter / kFBN : d->inter / 64;
    p.a_blk = d->a_layout == MOE_ACT_BLOCKED16;
    p.sh_a_blk = 0;       // the shared expert reads its rows of x in place
    p.out_blk = h_blk;
    st = launch_stage(p, f32, fp8, kUp, sk, parts, stream);
    if (st != MOE_OK) return st;
  }
  if (down) {
    p.a = h;
    p.a_rows = nullptr;
    p.w = w2;
    p.s = s2;
    p.out = y;
    p.sh_a = sh_h;
    p.sh_w = se ? se->w2 : nullptr;
    p.sh_s = se ? se->s2 : nullptr;
    p.sh_out = se ? se->y : nullptr;
    p.n_w_rows = d->hidden;
    p.K = d->inter;
    p.n_out = d->hidden;
    p.n_tiles_n = f32 ? d->hidden / kFBN : d->hidden / 128;
    p.a_blk = p.sh_a_blk = h_blk;  // h
    p.out_blk = 0;                // y rows are read by the combine
    st = launch_stage(p, f32, fp8, kDown, sk, parts, stream);
  }
  return st;
}

MOE_API moe_status_t moe_pack_weights(int n_groups, int hidden, int inter, moe_dtype_t w_dt, const void* w13,
                                      const void* w2, void* w13_packed, void* w2_packed, hipStream_t stream) {
  if (n_groups < 0 || hidden < 1 || inter < 1) return MOE_ERR_INVALID_ARG;
  if (w_dt != MOE_BF16 && w_dt != MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
  if (hidden % 128 || inter % 128) return MOE_ERR_UNSUPPORTED;
  if (n_groups == 0) return MOE_OK;
  const bool fp8 = w_dt == MOE_FP8_E4M3;
  const int64_t eb = fp8 ? 1 : 2;
  const int64_t bytes13 = int64_t(n_groups) * 2 * inter * hidden * eb, bytes2 = int64_t(n_groups) * hidden * inter * eb;
  if ((w13 == nullptr) != (w13_packed == nullptr) || (w2 == nullptr) != (w2_packed == nullptr))
    return MOE_ERR_INVALID_ARG;
  for (const void* q : {w13, w2, static_cast<const void*>(w13_packed), static_cast<const void*>(w2_packed)})
    if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if ((w13 && w13 == w13_packed) || (w2 && w2 == w2_packed)) return MOE_ERR_INVALID_ARG;  // not in place
  const dim3 block(256);
  if (w13) {
    const int64_t n = bytes13 / 16;
    const dim3 grid(unsigned(std::min<int64_t>((n + 255) / 256, 65536)));
    hipLaunchKernelGGL(pack_weights_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(w13),
                       static_cast<uint4*>(w13_packed), n, int(kUp), int(fp8), 2 * inter, hidden, inter, inter / 64);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  if (w2) {
    const int64_t n = bytes2 / 16;
    const dim3 grid(unsigned(std::min<int64_t>((n + 255) / 256, 65536)));
    hipLaunchKernelGGL(pack_weights_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(w2),
                       static_cast<uint4*>(w2_packed), n, int(kDown), int(fp8), hidden, inter, hidden, hidden / 128);
  }
  return launch_status();
}
