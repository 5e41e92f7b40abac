// Grouped-GEMM internals shared by the kernel translation units
// (gemm_wide.hip, gemm_bf16.hip, gemm_fp8.hip, gemm_w8a8.hip) and the host code in
// grouped_gemm.hip. Internal header.
#pragma once

#include <algorithm>
#include <type_traits>

#include "moe_common.hpp"

namespace moe {

// Weighted scatter from the down projection (moe_scatter_t): rows whose token
// has exactly one row of this GPU and no shared-expert row go to out.
struct ScatterArgs {
  const int32_t* row_token;   // [rows] token of each routed row
  const int32_t* row_of;      // [N, K]
  const float* w;             // [N, K] router weights
  uint16_t* out;              // [N, H] bf16 (nullptr: no scatter)
  int64_t n_rows;             // entries in [0, n_rows) are this GPU's rows
  int K, self_lo, self_hi;
};

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
  int interleave;             // W8A8: ranges of many whole tiles interleave them (prefill-sized launches)
  int a_blk, sh_a_blk;        // routed / shared activations in the 16-row blocked layout
  int out_blk;                // outputs (routed and shared) in the 16-row blocked layout
  const int32_t* a_rows;      // routed input row r is row a_rows[r] of a (nullptr: row r)
  int a_nrows;                // rows of a when gathering
  // W8A8: a (and sh_a) are e4m3 codes with one fp32 scale per row and 128
  // columns in as / sh_as; the up projection writes h as codes (out, sh_out)
  // and scales (out_s, sh_out_s); the down projection writes bf16
  const float* as;
  const float* sh_as;
  float* out_s;
  float* sh_out_s;
  ScatterArgs sc;             // down projection only
};

// Launchers of the four MFMA kernel families (each in its own translation
// unit): the main kernel of the stage and its fix-up kernel on `stream`.
moe_status_t launch_wide(const GemmArgs& p, int kind, float* parts, hipStream_t stream);
moe_status_t launch_bf16(const GemmArgs& p, int kind, float* parts, hipStream_t stream);
moe_status_t launch_fp8(const GemmArgs& p, int kind, float* parts, hipStream_t stream);
moe_status_t launch_w8a8(const GemmArgs& p, int kind, float* parts, hipStream_t stream);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kMaxGemmThreads = 512;  // the W8A16 decode and the wide kernels' workgroups
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
  int full_start[kMaxGroups + 2];  // wide kernel: exclusive prefix of the groups' full-row-tile tiles
  int m[kMaxGroups + 1];
  int goff[kMaxGroups + 1];  // compact layout: each group's first row (the shared expert: 0)
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
      sh.goff[nsh + g] = int(lo);
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
    if (nsh) {
      sh.m[0] = p.sh_rows;
      sh.goff[0] = 0;
    }
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
  // does all the work; small groups are cheap ragged tiles there); a launch
  // without the wide kernel (wide_min == kNoWide) never qualifies
  const int wide_min = p.wide_min != kNoWide && sh.wide_tiles >= p.wide_min_tiles ? 1 : kNoWide;
  for (int g = tid; g < Gt; g += NT) {
    const int m = sh.m[g];
    const bool mine = (m >= wide_min) == wide;
    sh.tile_start[g] = mine ? (m + bm - 1) / bm * ntn : 0;
    if (wide) sh.full_start[g] = mine ? m / bm * ntn : 0;
  }
  __syncthreads();
  const int total = block_scan_lds<false, NT>(sh.tile_start, Gt, sh.tmp);
  if (wide) {
    const int full = block_scan_lds<false, NT>(sh.full_start, Gt, sh.tmp);
    if (tid == 0) sh.full_start[Gt] = full;
  }
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

// Tile order of the wide kernel, in two phases. First every group's full
// row tiles (bm rows each), the N tiles cut into blocks of nbw as in
// decode_tile<true>: all these tiles cost the same, so the workgroups of an
// XCD, which take consecutive tiles, stay in step through a round and keep
// sharing the operand slabs in their L2. Then the groups' last, partial row
// tiles (rows m % bm), N tiles fastest. tile_start (all tiles) minus
// full_start (full-row-tile tiles) is the prefix of the partial tiles.
__device__ __forceinline__ Tile decode_tile_wide(const GemmArgs& p, int bm, int ntn, const Sched& sh, int t) {
  const int nsh = p.sh_rows > 0 ? 1 : 0;
  const int Gt = p.G + nsh;
  const int A = sh.full_start[Gt];
  const bool full = t < A;
  const int u = full ? t : t - A;
  int lo = 0, hi = Gt;  // last q with start[q] <= u
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    const int st = full ? sh.full_start[mid] : sh.tile_start[mid] - sh.full_start[mid];
    if (st <= u) lo = mid;
    else hi = mid;
  }
  Tile tl;
  tl.shared = lo < nsh;
  tl.g = tl.shared ? 0 : lo - nsh;
  tl.we = tl.g;
  const int m = sh.m[lo];
  const int mf = m / bm;  // full row tiles of the group
  tl.mtiles = (m + bm - 1) / bm;
  if (full) {
    const int local = u - sh.full_start[lo];
    const int nbw = ntn % 4 == 0 ? 4 : (ntn % 2 == 0 ? 2 : 1);
    const int blk = local / (nbw * mf), rem = local % (nbw * mf);
    tl.nt = blk * nbw + rem % nbw;
    tl.r0 = (rem / nbw) * bm;
    tl.nrows = bm;
  } else {
    tl.nt = u - (sh.tile_start[lo] - sh.full_start[lo]);
    tl.r0 = mf * bm;
    tl.nrows = m - tl.r0;
  }
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
      const int64_t base = sh.goff[tl.shared ? 0 : (p.sh_rows > 0 ? 1 : 0) + tl.g];  // (set by build_schedule)
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

// silu(g) = g / (1 + e^-g), the division as a product with the hardware
// reciprocal (1 ulp): a correctly rounded division is a ten-instruction
// sequence, and the result is rounded to bf16 (or compared at fp32 tolerance)
// right after. g -> -inf: e^-g = inf, rcp(inf) = 0, the product -0 as for the
// division.
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// e4m3fn x 8 (two dwords) -> bf16 x 8 of code * scale: exact decode to fp32
// (v_cvt_pk_f32_fp8), one fp32 multiply by the 128x128 block scale, one RNE
// rounding to bf16. (v_cvt_scalef32_pk_bf16_fp8 would apply only the
// power-of-two exponent of a scale, which block scales are not.)
__device__ __forceinline__ bf16x8_t fp8x8_dequant(uint32_t w0, uint32_t w1, float s) {
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

// Data-parallel + stream-K split (the decode kernels): of the launch's
// n_tiles tiles (nc chunks each) over G workgroups, workgroup range r first
// takes `whole` = n_tiles / G consecutive whole tiles, [r whole nc, (r + 1)
// whole nc), and then an even share of the remaining tiles' iterations,
// rem_base + [sk_start(r, rem, G), sk_start(r + 1, rem, G)). Only the second
// part ever cuts a tile, so partial sums number about 2 G fewer than with
// stream-K over everything, and during the first part all workgroups are at
// the same chunk index of their tiles, so the tiles of one expert (which sit
// in neighbouring ranges on one XCD) read each activation chunk at about the
// same time and the XCD's L2 serves the repeats. The remainder part costs
// partial sums and a fix-up, and with one whole tile per range it is over a
// third of the work, its ranges starting at different chunks of their tiles
// (no shared activation reads). So when ceil(n_tiles / G) <= 4 whole tiles
// per range fit on at least 3/4 of the grid, the split takes only whole
// tiles, on ceil(n_tiles / ceil(n_tiles / G)) ranges (the last takes what is
// left): no tile is cut (kimi_k2_ep8 up projection, two tiles per range: 394
// -> 373 us; dsv3_decode_ep8 down projection, four tiles per range on 224
// workgroups: 187 -> 175 us; kimi_k2_ep8 W8A8 down: 242 -> 231 us). With more
// whole tiles per range the remainder is kept: it balances tiles of unequal
// cost (whole tiles only made the W8A8 prefill up projection 5% slower,
// twelve tiles per range).
struct DpSk {
  int G;             // ranges (workgroups used)
  int whole;         // whole tiles per range, taken first
  int64_t rem_base;  // first iteration of the remainder tiles
  int64_t rem;       // iterations of the remainder tiles
};
__device__ inline DpSk dpsk_split(int n_tiles, int nc, int max_grid) {
  DpSk d;
  d.G = sk_grid(int64_t(n_tiles) * nc, max_grid);
  if (n_tiles % d.G != 0 && n_tiles > d.G) {
    const int w = (n_tiles + d.G - 1) / d.G;
    const int g2 = (n_tiles + w - 1) / w;
    if (w <= 4 && 4 * g2 >= 3 * d.G) {
      d.G = g2;
      d.whole = w;
      d.rem_base = int64_t(n_tiles) * nc;
      d.rem = 0;
      return d;
    }
  }
  d.whole = n_tiles / d.G;
  d.rem_base = int64_t(d.whole) * d.G * nc;
  d.rem = int64_t(n_tiles) * nc - d.rem_base;
  return d;
}

// Range of workgroup b (b < G): the workgroups of an XCD (b % kXcds) take
// consecutive ranges, G / kXcds of them (one more on the first G % kXcds
// XCDs), so neighbouring tiles share that XCD's L2.
__device__ inline int xcd_range(int b, int G) {
  const int x = b % kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

// Partial slot of workgroup b: 0 for its first tile, 1 for its last.
__device__ inline float* sk_slot(float* parts, int b, int slot) {
  return parts + (size_t(b) * 2 + slot) * kPartFloats;
}

// Fix-up records of the stream-K decode kernels, so that a fix-up rebuilds no
// schedule. After the 2 x grid partial slots (slot_floats each): [0] the
// ranges G, [1..2] rem_base, [3..4] rem (int64 halves), written by
// workgroup 0; from kSkMetaRecs, one record per range j, written by range j:
// [0] the tile whose first cut is the boundary after range j (-1: none), [1]
// its N tile, [2] shared, [3] rows, [4] b_lo, [5] b_hi (the ranges over it),
// then its physical rows.
constexpr int kSkRecRows = 96;  // tile rows of the decode kernels (bf16 64, fp8 96)
constexpr int kSkRecInts = 8 + kSkRecRows;
constexpr int kSkMetaRecs = 8;
constexpr int kSkMetaInts = kSkMetaRecs + 256 * kSkRecInts;  // grids of at most 256 ranges

__device__ __forceinline__ int* sk_meta(float* parts, size_t slot_floats, int grid) {
  return reinterpret_cast<int*>(parts + size_t(2) * grid * slot_floats);
}

// Main kernel, before its ranges: the header, and no record for range rng
// until sk_write_rec sets one.
__device__ __forceinline__ void sk_meta_begin(int* meta, const DpSk& sp, int rng) {
  if (threadIdx.x == 0) {
    if (blockIdx.x == 0) {
      meta[0] = sp.G;
      meta[1] = int(uint32_t(uint64_t(sp.rem_base)));
      meta[2] = int(uint32_t(uint64_t(sp.rem_base) >> 32));
      meta[3] = int(uint32_t(uint64_t(sp.rem)));
      meta[4] = int(uint32_t(uint64_t(sp.rem) >> 32));
    }
    meta[kSkMetaRecs + rng * kSkRecInts] = -1;
  }
}

// Whether remainder range [i0, i1) ends inside a tile whose chunk 0 it
// holds: the boundary after it is that tile's first cut.
__device__ __forceinline__ bool sk_owns_cut(int64_t i0, int64_t i1, int nchunks) {
  return i0 < i1 && i1 % nchunks != 0 && i0 <= i1 / nchunks * nchunks;
}

// Range rng's record of tile t, a tile of the run that starts at tile t_run
// (tl, whose rows are in sh.rowmap: every tile of a run has the same rows).
template <int NT>
__device__ __forceinline__ void sk_write_rec(int* meta, int rng, int t, int t_run, const Tile& tl, const Sched& sh,
                                             int b_hi) {
  int* rec = meta + kSkMetaRecs + rng * kSkRecInts;
  if (threadIdx.x == 0) {
    rec[0] = t;
    rec[1] = tl.nt + (t - t_run);
    rec[2] = tl.shared;
    rec[3] = tl.nrows;
    rec[4] = rng;
    rec[5] = b_hi;
  }
  for (int i = threadIdx.x; i < tl.nrows; i += NT) rec[8 + i] = sh.rowmap[i];
}

// Fix-up side: the record of the boundary after range j (false: none).
struct SkRec {
  int t, b_lo, b_hi;
  Tile tl;
  DpSk sp;
};
__device__ __forceinline__ bool sk_read_rec(const int* meta, int j, int bm, SkRec& r) {
  r.sp.G = __builtin_amdgcn_readfirstlane(meta[0]);
  if (j + 1 >= r.sp.G) return false;  // boundaries lie between ranges 0 .. G - 1
  const int* rec = meta + kSkMetaRecs + j * kSkRecInts;
  r.t = __builtin_amdgcn_readfirstlane(rec[0]);
  if (r.t < 0) return false;
  r.sp.rem_base = int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(meta[1]))) |
                          uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(meta[2]))) << 32);
  r.sp.rem = int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(meta[3]))) |
                     uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(meta[4]))) << 32);
  r.sp.whole = 0;
  r.tl = Tile{};
  r.tl.nt = __builtin_amdgcn_readfirstlane(rec[1]);
  r.tl.shared = __builtin_amdgcn_readfirstlane(rec[2]) != 0;
  r.tl.nrows = min(max(__builtin_amdgcn_readfirstlane(rec[3]), 0), bm);
  r.b_lo = __builtin_amdgcn_readfirstlane(rec[4]);
  r.b_hi = min(__builtin_amdgcn_readfirstlane(rec[5]), r.sp.G - 1);
  return true;
}
// The record's physical rows into sh.rowmap (-1 past the tile's rows). All
// threads must call it.
template <int NT>
__device__ __forceinline__ void sk_read_rows(const int* meta, int j, int bm, int nrows, Sched& sh) {
  const int* rec = meta + kSkMetaRecs + j * kSkRecInts;
  for (int i = threadIdx.x; i < bm; i += NT) sh.rowmap[i] = i < nrows ? rec[8 + i] : -1;
  __syncthreads();
}

// The token of routed row phys when its down-projection row is that token's
// whole combine (exactly one of its K entries is a row of this GPU, and it
// has no shared-expert row), with that entry's weight in w; else -1. The rule
// is moe_combine's own (an entry is kept when its row lies in [0, n_rows)).
__device__ __forceinline__ int scatter_token(const ScatterArgs& sc, int64_t phys, float& w) {
  const int t = sc.row_token[phys];
  if (t < 0 || (t >= sc.self_lo && t < sc.self_hi)) return -1;
  int n = 0;
  float wk = 0.f;
  for (int k = 0; k < sc.K; ++k) {
    const int r = sc.row_of[size_t(t) * sc.K + k];
    if (r >= 0 && r < sc.n_rows) {
      ++n;
      wk = sc.w[size_t(t) * sc.K + k];
    }
  }
  w = wk;
  return n == 1 ? t : -1;
}

// Four consecutive down-projection outputs at column col of row `row`: y
// values rounded to bf16, or (scat: row is the token's output row) as
// moe_combine writes a token with one kept row, round(w * bf16(y)) with the
// product formed as fmaf(w, y, 0).
__device__ __forceinline__ void store_y4(uint16_t* row, bool scat, float sw, int col, float v0, float v1, float v2,
                                         float v3) {
  const uint32_t p0 = pack_bf16x2(v0, v1), p1 = pack_bf16x2(v2, v3);
  if (!scat) {
    *reinterpret_cast<uint2*>(row + col) = make_uint2(p0, p1);
    return;
  }
  const float y0 = __uint_as_float(p0 << 16), y1 = __uint_as_float(p0 & 0xffff0000u);
  const float y2 = __uint_as_float(p1 << 16), y3 = __uint_as_float(p1 & 0xffff0000u);
  *reinterpret_cast<uint2*>(row + col) = make_uint2(pack_bf16x2(fmaf(sw, y0, 0.f), fmaf(sw, y1, 0.f)),
                                                    pack_bf16x2(fmaf(sw, y2, 0.f), fmaf(sw, y3, 0.f)));
}

// Epilogue of 32-row block b of a tile (four consecutive output columns never
// straddle a 32-column block).
template <int KIND>
__device__ __forceinline__ void ffn_epilogue_block(const f32x16_t& acc, const Tile& tl, int b, const Sched& sh,
                                                   uint16_t* out, int n_out, int wv, int lr, int lh, bool oblk,
                                                   const ScatterArgs& sc) {
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
    // (y rows are row-major)
    float sw = 0.f;
    const int st = sc.out != nullptr && !tl.shared ? scatter_token(sc, phys, sw) : -1;
    uint16_t* yrow = st >= 0 ? sc.out + size_t(st) * n_out : orow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = tl.nt * 128 + 32 * wv + 8 * q + 4 * lh;
      store_y4(yrow, st >= 0, sw, col, acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
  }
}

template <int KIND, int NBMAX>
__device__ __forceinline__ void ffn_epilogue(const f32x16_t (&acc)[NBMAX], const Tile& tl, int nb, const Sched& sh,
                                             uint16_t* out, int n_out, int wv, int lr, int lh, bool oblk,
                                             const ScatterArgs& sc) {
#pragma unroll
  for (int b = 0; b < NBMAX; ++b)
    if (b < nb) ffn_epilogue_block<KIND>(acc[b], tl, b, sh, out, n_out, wv, lr, lh, oblk, sc);
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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

// One wide tile's accumulators: 4 waves x 2 weight blocks x 8 activation
// blocks x 16 registers x 64 lanes.
constexpr int kWidePart = 4 * 2 * 8 * 16 * kWave;
// [wave pair][wave in pair][block][quad q][lane][4 floats]: registers
// 4q..4q+3 of one accumulator tile, 16 bytes per lane, 1 KiB contiguous per
// wave access
__device__ __forceinline__ int wide_part_idx(int wv, int a, int b, int q, int lane) {
  return ((((wv * 2 + a) * 8 + b) * 4 + q) * kWave + lane) * 4;
}
// After the wide kernel's kWideGrid partial slots: words its main kernel
// leaves for the fix-up, so that the fix-up rebuilds no schedule. [0] the
// number of K-split tiles (0: none), [1] their ranges each; from
// kWideMetaRecs, one record per split tile: N tile, shared, rows, then the
// tile's physical rows.
constexpr int kWideRec = 8 + kWM;
constexpr int kWideMetaRecs = 16;
constexpr int kWideMetaInts = kWideMetaRecs + kWideGrid * kWideRec;
__device__ __forceinline__ int* wide_meta(float* parts) { return reinterpret_cast<int*>(parts + size_t(kWideGrid) * kWidePart); }


constexpr int kF8BM = 96;                                           // activation rows per tile
constexpr int kF8MB = kF8BM / 32;                                   // MFMA row blocks per tile
constexpr int kF8Waves = 8;                                         // waves per workgroup
constexpr int kF8Threads = kF8Waves * kWave;
constexpr int kF8NB = kF8Waves / 2;                                 // N blocks per tile
constexpr int kF8Grid = 256;                                        // 1 resident workgroup x 256 CUs
constexpr int kF8PartFloats = kF8Waves * 2 * kF8MB * 16 * kWave;   // one workgroup's accumulators (192 KiB)
static_assert(kF8Threads <= kMaxGemmThreads, "schedule scratch holds one entry per thread");
static_assert(kBfGrid <= 256 && kF8Grid <= 256 && kBfBM <= kSkRecRows && kF8BM <= kSkRecRows,
              "fix-up records: one per range, a tile's rows each");

}  // namespace
}  // namespace moe
