// fp8 (e4m3 weights, W8A16) stream-K grouped-GEMM kernel; see the kernel comment.
#include "gemm_common.hpp"

namespace moe {
namespace {

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
  // through the compiler's builtin, so its wait analysis sees the copies and
  // waits for them before the LDS reads: the completion of an LDS copy is not
  // ordered with the loads into registers, so the counted waits below alone
  // do not guarantee it - with them alone the W8A8 kernel read stale rows now
  // and then. The buffer form of the LDS copy is not used, its LDS addressing
  // on this chip - scalar offset, destinations above 64 KiB - not being
  // established.)
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
      __builtin_amdgcn_global_load_lds(at<void>(xc_, 0, xoff[q]), (lds_ptr_t)((XBUF_) + (kF8Waves * q + wv) * 512), \
                                       16, 0, 0);                                                           \
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
          if (ta_.nt < p.n_tiles_n) ffn_epilogue<KIND, NB>(acc[a], ta_, NB, sh, out, p.n_out, wq, lr, lh, p.out_blk, p.sc); \
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
  const DpSk sp = dpsk_split(n_tiles, nchunks, kF8Grid);
  if (int(blockIdx.x) >= sp.G) return;  // uniform
  const int G = sp.G;
  const int rng = xcd_range(int(blockIdx.x), G);
  int* meta = sk_meta(parts, kF8PartFloats, kF8Grid);
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
      const Tile tl = decode_tile(p, kF8BM, ntn4, sh, t);
      build_rowmap<kF8Threads>(p, tl, kF8BM, sh, true);
      const int n = tl.mtiles == 1 ? min(t_last - t + 1, ntn4 - tl.nt) : 1;
      if (rec_cut && t_last < t + n)  // uniform
        sk_write_rec<kF8Threads>(meta, rng, t_last, t, tl, sh,
                         sk_owner(int64_t(t_last + 1) * nchunks - 1 - sp.rem_base, sp.rem, G));
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
  const int nchunks = p.K / kKC;
  const int j = blockIdx.x, m = blockIdx.y / kF8MB, b = blockIdx.y % kF8MB;
  // the tile and its ranges from the record range j left (no schedule rebuilt;
  // the whole-tile parts never cut a tile)
  const int* meta = sk_meta(const_cast<float*>(parts), kF8PartFloats, kF8Grid);
  SkRec r;
  if (!sk_read_rec(meta, j, kF8BM, r)) return;  // uniform: the boundary after range j is no tile's first cut
  const DpSk sp = r.sp;
  const int G = sp.G, t = r.t, b_lo = r.b_lo, b_hi = r.b_hi;
  Tile tl = r.tl;
  if (b * 32 >= tl.nrows || kF8NB * tl.nt + m >= p.n_tiles_n) return;  // uniform: no rows / no such N block
  sk_read_rows<kGemmThreads>(meta, j, kF8BM, tl.nrows, sh);
  f32x16_t acc[1];
  sum_partials(
      acc, b_lo, b_hi,
      [&](int w) -> const float* {
        const int64_t s0 = sp.rem_base + sk_start(w, sp.rem, G), s1 = sp.rem_base + sk_start(w + 1, sp.rem, G);
        return s0 < s1 ? f8_slot(const_cast<float*>(parts), w, int(s0 / nchunks) == t ? 0 : 1) : nullptr;
      },
      [&](int, int q) { return f8_part_idx(m / 2 * 4 + wv, m % 2, b, q, lane); });
  tl.nt = kF8NB * tl.nt + m;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  ffn_epilogue_block<KIND>(acc[0], tl, b, sh, out, p.n_out, wv, lr, lh, p.out_blk, p.sc);
}

}  // namespace

moe_status_t launch_fp8(const GemmArgs& p, int kind, float* parts, hipStream_t stream) {
  const dim3 grid(kF8Grid), block(kF8Threads);
  if (kind == kUp) {
    if (p.packed) hipLaunchKernelGGL((ffn_fp8_kernel<kUp, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_fp8_kernel<kUp, false>), grid, block, 0, stream, p, parts);
  } else {
    if (p.packed) hipLaunchKernelGGL((ffn_fp8_kernel<kDown, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_fp8_kernel<kDown, false>), grid, block, 0, stream, p, parts);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 fix_grid(kF8Grid - 1, kF8NB * kF8MB);
  if (kind == kUp) hipLaunchKernelGGL((ffn_fp8_fixup_kernel<kUp>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_fp8_fixup_kernel<kDown>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  return launch_status();
}

}  // namespace moe
