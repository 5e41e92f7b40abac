// bf16 stream-K grouped-GEMM kernel (decode-shaped groups); see the kernel comment.
#include "gemm_common.hpp"

namespace moe {
namespace {

// Finishes the tiles of ffn_bf16_kernel cut by a stream-K range boundary:
// block (j, m * kBfMB + b) looks at the boundary between ranges j and j+1;
// where it is a tile's first cut (range j left a record of the tile), it
// sums, for the tile's N block m and 32-row block b, the partials in range
// order (one wave per 32 weight rows of the N block, i.e. the partials of the
// main kernel's waves 4 m .. 4 m + 3) and runs that block's epilogue.
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nchunks = p.K / kKC;
  const int j = blockIdx.x, m = blockIdx.y / kBfMB, b = blockIdx.y % kBfMB;
  // the tile and its ranges from the record range j left (no schedule rebuilt)
  const int* meta = sk_meta(const_cast<float*>(parts), kPartFloats, kBfGrid);
  SkRec r;
  if (!sk_read_rec(meta, j, kBfBM, r)) return;  // uniform: the boundary after range j is no tile's first cut
  const DpSk sp = r.sp;
  const int G = sp.G, t = r.t, b_lo = r.b_lo, b_hi = r.b_hi;
  Tile tl = r.tl;
  if (b * 32 >= tl.nrows || kBfNB * tl.nt + m >= p.n_tiles_n) return;  // uniform: no rows / no such N block
  sk_read_rows<kGemmThreads>(meta, j, kBfBM, tl.nrows, sh);
  f32x16_t acc[1];
  sum_partials(
      acc, b_lo, b_hi,
      [&](int w) -> const float* {
        const int64_t s0 = sp.rem_base + sk_start(w, sp.rem, G), s1 = sp.rem_base + sk_start(w + 1, sp.rem, G);
        return s0 < s1 ? sk_slot(const_cast<float*>(parts), w, int(s0 / nchunks) == t ? 0 : 1) : nullptr;
      },
      [&](int, int q) { return bf_part_idx(4 * m + wv, b, q, lane); });
  tl.nt = kBfNB * tl.nt + m;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  ffn_epilogue_block<KIND>(acc[0], tl, b, sh, out, p.n_out, wv, lr, lh, p.out_blk, p.sc);
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
        if (tk_.nt < p.n_tiles_n) ffn_epilogue<KIND, NB>(acc, tk_, NB, sh, out, p.n_out, wq, lr, lh, p.out_blk, p.sc); \
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
  const DpSk sp = dpsk_split(n_tiles, nchunks, kBfGrid);
  if (int(blockIdx.x) >= sp.G) return;  // uniform
  const int G = sp.G;
  const int rng = xcd_range(int(blockIdx.x), G);
  int* meta = sk_meta(parts, kPartFloats, kBfGrid);
  sk_meta_begin(meta, sp, rng);
  // the range's whole tiles first, then its share of the remainder
  for (int part = 0; part < 2; ++part) {
    const int64_t i0 = part == 0 ? int64_t(rng) * sp.whole * nchunks : sp.rem_base + sk_start(rng, sp.rem, G);
    const int64_t i1 = part == 0 ? min(int64_t(rng + 1) * sp.whole, int64_t(n_tiles)) * nchunks
                                 : sp.rem_base + sk_start(rng + 1, sp.rem, G);
    if (i0 >= i1) continue;  // uniform
    const int t_first = int(i0 / nchunks), t_last = int((i1 - 1) / nchunks);
    const bool rec_cut = part == 1 && sk_owns_cut(i0, i1, nchunks);  // the fix-up's record of tile t_last
    for (int t = t_first; t <= t_last;) {
      const Tile tl = decode_tile(p, kBfBM, ntn2, sh, t);
      build_rowmap<kBfThreads>(p, tl, kBfBM, sh, true);
      // a run: with one row tile the group's next tiles are its next N tiles
      // (same activation rows)
      const int n = tl.mtiles == 1 ? min(t_last - t + 1, ntn2 - tl.nt) : 1;
      if (rec_cut && t_last < t + n)  // uniform
        sk_write_rec<kBfThreads>(meta, rng, t_last, t, tl, sh,
                         sk_owner(int64_t(t_last + 1) * nchunks - 1 - sp.rem_base, sp.rem, G));
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
}

}  // namespace

moe_status_t launch_bf16(const GemmArgs& p, int kind, float* parts, hipStream_t stream) {
  const dim3 grid(kBfGrid), block(kBfThreads);
  if (kind == kUp) {
    if (p.packed) hipLaunchKernelGGL((ffn_bf16_kernel<kUp, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_bf16_kernel<kUp, false>), grid, block, 0, stream, p, parts);
  } else {
    if (p.packed) hipLaunchKernelGGL((ffn_bf16_kernel<kDown, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_bf16_kernel<kDown, false>), grid, block, 0, stream, p, parts);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 fix_grid(kBfGrid - 1, kBfNB * kBfMB);
  if (kind == kUp) hipLaunchKernelGGL((ffn_fixup_kernel<kUp>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_fixup_kernel<kDown>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  return launch_status();
}

}  // namespace moe
