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
// every workgroup from the device counts. A tile is (expert, row block, N
// block); empty experts produce no tiles. Four kernel families share that
// scheduler (gemm_common.hpp), each in its own translation unit:
//  - ffn_bf16_kernel (gemm_bf16.hip): decode-shaped groups, bf16 weights;
//    tiles of 64 rows x 256 weight rows on 8-wave workgroups, stream-K over
//    (tile, 128-deep chunk) iterations, weights streamed from HBM into
//    registers, activations copied into LDS;
//  - ffn_fp8_kernel (gemm_fp8.hip): fp8 e4m3 weights with 128 x 128 scales and
//    bf16 activations (W8A16): 96 rows x 512 weight rows on 8 waves, each code
//    decoded exactly, scaled and rounded once to bf16 in registers;
//  - ffn_w8a8_kernel (gemm_w8a8.hip): fp8 weights and fp8 activations with
//    1 x 128 scales: the same tiles on 4 waves, fp8 MFMA with the block scales
//    applied per 128-deep chunk, h quantized in the up projection's epilogue;
//  - ffn_wide_kernel (gemm_wide.hip): groups with many rows: 256 x 256 tiles on
//    8 waves (two per SIMD), weights in a register ring, activations staged
//    through registers into LDS, full-row tiles first, remainder tiles split
//    along K.
// Tiles cut by a stream-K or K-split boundary leave fp32 partial sums that a
// fix-up kernel adds in a fixed order (deterministic) before the epilogue.
// MFMA with the weights as the A operand (32 weight rows) and the activations
// as the B operand; each wave owns 32-row weight blocks (up: 16 gate rows and
// the 16 matching up rows, so the SwiGLU pairs land in one lane).
//
// fp32 activations + fp32 weights (small parity problems) use a plain SIMT
// kernel with the same scheduler (below).
#include "gemm_common.hpp"

namespace moe {
namespace {

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

static bool is_w8a8(const moe_ggemm_desc_t* d) { return d->act_dt == MOE_FP8_E4M3 && d->w_dt == MOE_FP8_E4M3; }

static bool ggemm_desc_supported(const moe_ggemm_desc_t* d) {
  const bool f32 = d->act_dt == MOE_F32 && d->w_dt == MOE_F32;
  const bool bf16 = d->act_dt == MOE_BF16 && (d->w_dt == MOE_BF16 || d->w_dt == MOE_FP8_E4M3);
  const bool w8a8 = is_w8a8(d);
  if (!f32 && !bf16 && !w8a8) return false;
  if (w8a8) {
    if (d->a_layout != MOE_ACT_ROWS) return false;
    // scale offsets are 32-bit byte offsets: rows * (K / 128) * 4 < 2^32
    const int64_t kmax = std::max(d->hidden, d->inter) / 128;
    const int64_t srows = std::max<int64_t>(d->rows, d->a_rows ? d->a_nrows : 0);
    if (srows * kmax * 4 >= (int64_t(1) << 32)) return false;
  }
  if (d->hidden % 128 || d->inter % 128) return false;
  if (d->n_groups > kMaxGroups) return false;
  if (d->layout == MOE_LAYOUT_PADDED && d->n_src > kGemmMaxSrc) return false;
  if (d->rows >= (int64_t(1) << 31)) return false;
  if (d->shared && d->shared->rows >= (1 << 30)) return false;
  if (f32 && d->w_format == MOE_W_PACKED) return false;
  if (f32 && d->a_layout != MOE_ACT_ROWS) return false;
  // gathering: row-major rows, 32-bit byte offsets (decode-shaped kernels)
  if (d->a_rows && (f32 || d->a_layout != MOE_ACT_ROWS ||
                    d->a_nrows > (int64_t(1) << 32) / (int64_t(d->hidden) * (w8a8 ? 1 : 2))))
    return false;
  return true;
}

// h codes of W8A8: [rows, I] bytes, then the scales [rows, I / 128]
static size_t h_codes_bytes(const moe_ggemm_desc_t* d, int64_t rows) {
  return align_up(size_t(rows) * size_t(d->inter), 256);
}

// h [rows, I]: fp32 row-major, or bf16 in the 16-row blocked layout (rows
// rounded up to 16), or W8A8 codes and scales
static size_t h_bytes(const moe_ggemm_desc_t* d, int64_t rows) {
  if (is_w8a8(d)) return h_codes_bytes(d, rows) + align_up(size_t(rows) * size_t(d->inter / 128) * 4, 256);
  const size_t el = d->act_dt == MOE_F32 ? 4 : 2;
  if (d->act_dt != MOE_F32) rows = (rows + 15) / 16 * 16;
  return align_up(size_t(rows) * size_t(d->inter) * el, 256);
}

static size_t parts_bytes(const moe_ggemm_desc_t* d) {
  // shared by the wide and the stream-K kernels, which run one after the other
  const size_t sk = (d->w_dt == MOE_FP8_E4M3 ? size_t(2) * kF8Grid * kF8PartFloats : size_t(2) * kBfGrid * kPartFloats) +
                    kSkMetaInts;
  const size_t wide = size_t(kWideGrid) * kWidePart + kWideMetaInts;
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
static moe_status_t launch_stage(const GemmArgs& p, bool f32, bool fp8, bool w8a8, int kind, bool sk, float* parts,
                                 hipStream_t stream) {
  if (w8a8) return launch_w8a8(p, kind, parts, stream);
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
    // the wide kernel's partials are finished (by its fix-up kernel) before
    // the stream-K kernel reuses the buffer
    const moe_status_t st = launch_wide(p, kind, parts, stream);
    if (st != MOE_OK || !sk) return st;
  }
  return fp8 ? launch_fp8(p, kind, parts, stream) : launch_bf16(p, kind, parts, stream);
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
  const bool w8a8 = is_w8a8(d);
  const bool up = d->stage != MOE_GG_DOWN, down = d->stage != MOE_GG_UP;
  auto aligned4 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; };
  if (routed) {
    if (d->layout == MOE_LAYOUT_COMPACT && !group_off) return MOE_ERR_INVALID_ARG;
    if (d->layout == MOE_LAYOUT_PADDED && !counts) return MOE_ERR_INVALID_ARG;
    if (up && (!a || !w13 || !aligned16(a) || !aligned16(w13))) return MOE_ERR_INVALID_ARG;
    if (down && (!y || !w2 || !aligned16(y) || !aligned16(w2))) return MOE_ERR_INVALID_ARG;
    if (fp8 && ((up && !s13) || (down && !s2))) return MOE_ERR_INVALID_ARG;
    if (w8a8 && up && (!d->a_scales || !aligned4(d->a_scales))) return MOE_ERR_INVALID_ARG;
  }
  if (se) {
    if (up && (!se->a || !se->w13 || !aligned16(se->a) || !aligned16(se->w13))) return MOE_ERR_INVALID_ARG;
    if (down && (!se->y || !se->w2 || !aligned16(se->y) || !aligned16(se->w2))) return MOE_ERR_INVALID_ARG;
    if (fp8 && ((up && !se->s13) || (down && !se->s2))) return MOE_ERR_INVALID_ARG;
    if (w8a8 && up && (!se->a_scales || !aligned4(se->a_scales))) return MOE_ERR_INVALID_ARG;
  }
  // weighted scatter from the down projection's epilogue (bf16 y only)
  const moe_scatter_t* sc = down && routed ? d->scatter : nullptr;
  if (sc) {
    if (f32) return MOE_ERR_UNSUPPORTED;
    if (!sc->row_token || !sc->row_of || !sc->topk_w || !sc->out || !aligned16(sc->out)) return MOE_ERR_INVALID_ARG;
    if (sc->n_tokens < 0 || sc->top_k < 1 || sc->top_k > 16 || sc->n_rows < 0) return MOE_ERR_INVALID_ARG;
    if (sc->self_lo < 0 || sc->self_hi < sc->self_lo || sc->self_hi > sc->n_tokens) return MOE_ERR_INVALID_ARG;
  }
  if (!ws || !aligned16(ws) || ws_bytes < moe_grouped_gemm_workspace(d)) return MOE_ERR_WORKSPACE;
  // the decode kernels address a tile's activation rows relative to its first
  // row: one expert's padded region must span fewer than 2^31 elements
  if (!f32 && d->layout == MOE_LAYOUT_PADDED &&
      (int64_t(d->n_src) * d->capacity + 16) * std::max(d->hidden, d->inter) >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;

  void* h = ws;
  void* sh_h = static_cast<char*>(ws) + h_bytes(d, d->rows);
  const int64_t sh_rows_ws = d->shared ? d->shared->rows : 0;
  float* parts = reinterpret_cast<float*>(static_cast<char*>(sh_h) + h_bytes(d, sh_rows_ws));
  // W8A8: the scales of h follow its codes
  float* h_s = w8a8 ? reinterpret_cast<float*>(static_cast<char*>(h) + h_codes_bytes(d, d->rows)) : nullptr;
  float* sh_h_s = w8a8 ? reinterpret_cast<float*>(static_cast<char*>(sh_h) + h_codes_bytes(d, sh_rows_ws)) : nullptr;
  GemmArgs p;
  p.sc = ScatterArgs{};
  p.as = p.sh_as = nullptr;
  p.out_s = p.sh_out_s = nullptr;
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
  const bool wide_ok = !f32 && !fp8 && !w8a8 && d->hidden % 256 == 0 && d->inter % 128 == 0 &&
                       d->policy != MOE_GEMM_STREAM_K;
  const bool force = d->policy == MOE_GEMM_WIDE;
  p.wide_min = wide_ok ? (force ? 1 : kWideMinRows) : kNoWide;
  const bool sk = !(wide_ok && force);  // forced wide leaves the stream-K kernel nothing
  // h (internal) in the 16-row blocked layout where the wide kernel may run
  // (its loads take 16 rows x 32 columns); row-major for the decode kernels,
  // whose loads take 4 rows x 128 columns
  const bool h_blk = wide_ok;
  p.wide_min_tiles = force ? 0 : kWideMinTiles;
  p.interleave = d->policy != MOE_GEMM_STREAM_K;
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
    p.as = d->a_scales;
    p.sh_as = se ? se->a_scales : nullptr;
    p.out_s = h_s;
    p.sh_out_s = sh_h_s;
    p.n_w_rows = 2 * d->inter;
    p.K = d->hidden;
    p.n_out = d->inter;
    p.n_tiles_n = f32 ? d->inter / kFBN : d->inter / 64;
    p.a_blk = d->a_layout == MOE_ACT_BLOCKED16;
    p.sh_a_blk = 0;       // the shared expert reads its rows of x in place
    p.out_blk = h_blk;
    st = launch_stage(p, f32, fp8, w8a8, kUp, sk, parts, stream);
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
    p.as = h_s;
    p.sh_as = sh_h_s;
    p.out_s = p.sh_out_s = nullptr;
    p.n_w_rows = d->hidden;
    p.K = d->inter;
    p.n_out = d->hidden;
    p.n_tiles_n = f32 ? d->hidden / kFBN : d->hidden / 128;
    p.a_blk = p.sh_a_blk = h_blk;  // h
    p.out_blk = 0;                // y rows are read by the combine
    if (sc) {
      p.sc.row_token = sc->row_token;
      p.sc.row_of = sc->row_of;
      p.sc.w = sc->topk_w;
      p.sc.out = static_cast<uint16_t*>(sc->out);
      p.sc.n_rows = sc->n_rows;
      p.sc.K = sc->top_k;
      p.sc.self_lo = sc->self_lo;
      p.sc.self_hi = sc->self_hi;
    }
    st = launch_stage(p, f32, fp8, w8a8, kDown, sk, parts, stream);
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
