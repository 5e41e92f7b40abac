// Wide-tile grouped-GEMM kernel (prefill-shaped groups); see the kernel comment.
#include "gemm_common.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ wide-tile kernel
// Groups with many rows (prefill, and decode with few experts per GPU) are
// compute-heavy: a weight block is used by hundreds of rows. Tile = 256
// weight rows x 256 activation rows for a workgroup of 8 waves, two per SIMD;
// wave w owns one 32-row block of the packed weight order (block w % 4 of the
// tile's 128-row weight block w / 4; up: 16 gate rows and the matching 16 up
// rows, so the SwiGLU pairs meet in one lane) against all 256 activation rows,
// a 32 x 256 fp32 accumulator block (8 MFMA 32x32 tiles, 128 registers). With
// two waves per SIMD, a wave waiting on memory or LDS leaves the matrix core
// to the other. (One wave per SIMD with 64 weight rows each, 256 accumulator
// registers, reads the activation fragments half as often but measured 1-2%
// slower on the prefill share.)
//
// Operands come from L2 and beyond at about 32 bytes per clock per compute
// unit when the matrix cores run flat out (64 KiB per 64-deep stage); so:
//  - the weights, private to a wave, go straight from memory into a
//    two-stage register ring (buffer loads, 1 KiB per wave instruction in the
//    packed order, each lane's 16 bytes exactly its MFMA operand), with no LDS
//    round trip;
//  - the activations, read by all 8 waves, are loaded two 64-deep stages
//    ahead into a two-slot register ring (16 bytes per lane per load; a 64-deep
//    stage puts 128 contiguous bytes of each row in one wave load, 8 rows x
//    128 bytes, whole 128-byte lines also for gathered token rows), and each
//    wave writes its share of a stage into a two-buffer LDS ring (2 x 32 KiB)
//    one stage before it is read.
// Every load is an ordinary load into registers, so the compiler's own wait
// counting stays exact; its analysis of LDS-writing loads (global_load_lds)
// forces full drains when such loads are mixed with loads into registers.
//
// The reduction order inside a 128-deep chunk follows the packed weight
// order: weight load i of chunk c holds, in lanes 0-31, k = 128 c + 64 (i / 4)
// + 8 (i % 4) .. + 8 and in lanes 32-63 the same + 32; the MFMA step using it
// reads the matching activation pieces. Each stage is four 16-deep steps;
// step j of stage s uses weight load 4 (s % 2) + j of chunk s / 2.
// LDS: a stage row is 128 bytes (8 pieces of 16); piece c of row r sits in
// slot c ^ ((r / 2) % 8), so the 16 rows a fragment read or a staging write
// serves together fall on 16 distinct 16-byte bank groups (0 conflicts).
//
// Per step a wave issues its MFMAs with the next step's fragment reads and
// its share of the loads in between; one barrier per stage (in the middle of
// its last step) publishes the next stage's activations.
constexpr int kAK = 64;                 // reduction depth of one stage
// (the LDS ring holds two stages: X[0], X[1])
constexpr int kAStage = kWM * kAK;      // elements of one activation stage (32 KiB)
// s_waitcnt operand: this wave's LDS operations done, vector memory not waited for
constexpr int kWaitLgkm0 = waitcnt_vm(63) & ~(15 << 8);

constexpr int kWideWaves = 8;
constexpr int kWideThreads = kWideWaves * kWave;

// Epilogue of 32-row activation block b of a wide tile from the accumulator
// tile of wave wv: weight block wv % 4 of the tile's 128-row block wv / 4 (up:
// the gate rows 0-15 and up rows 16-31 of 16 h columns; down: 32 output
// columns).
template <int KIND>
__device__ __forceinline__ void wide_epilogue_block(const GemmArgs& p, const Tile& tl, const Sched& sh, int b,
                                                     const f32x16_t& ac, int wv, int lr, int lh) {
  const int phys = sh.rowmap[32 * b + lr];
  if (phys < 0) return;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  const bool oblk = p.out_blk;
  uint16_t* orow = out + act_off(phys, 0, p.n_out, oblk);
  const int ntp = 2 * tl.nt + (wv >> 2);
  const int pw = wv & 3;
  if (KIND == kUp) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = silu_f(ac[4 * q + r]) * ac[4 * (q + 2) + r];
      const int col = ntp * 64 + 16 * pw + 8 * q + 4 * lh;
      *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
          make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
    }
  } else {
    // (y rows are row-major)
    float sw = 0.f;
    const int st = p.sc.out != nullptr && !tl.shared ? scatter_token(p.sc, phys, sw) : -1;
    uint16_t* yrow = st >= 0 ? p.sc.out + size_t(st) * p.n_out : orow;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = ntp * 128 + 32 * pw + 8 * q + 4 * lh;
      store_y4(yrow, st >= 0, sw, col, ac[4 * q], ac[4 * q + 1], ac[4 * q + 2], ac[4 * q + 3]);
    }
  }
}

// Output staging of whole tiles through LDS (the activation ring is free
// after the K loop). Stored straight from the accumulators, every wave
// instruction writes 16-byte pieces of 32 rows; such stores complete slowly,
// and a tile's first loads wait behind the previous tile's stores (the vector
// memory counter counts loads and stores in issue order). So a tile's outputs
// are staged as bf16 rows in LDS and stored as whole row pieces: 512
// contiguous bytes per y row (down), 64-byte row pieces of the blocked h
// layout, 1 KiB per wave instruction (up). Staging slots: 16-byte piece c of
// row r at slot c ^ (r % 16) (up, 256-byte rows) or c ^ (r % 32) (down,
// 512-byte rows), so that a wave's staging writes and row reads spread over
// the banks. The stores carry the non-temporal hint (measured 0.5% faster
// on the prefill share). (Deferring a tile's stores past the next tile's
// first loads, through 64 KiB more of LDS, measured no better.)

// Blocks [b0, b1) of the accumulators into a staging area: up, [128 rows]
// [128 h columns] per buffer (buf0: blocks 0-3, buf1: 4-7); down, [64 rows]
// [256 columns] per buffer (blocks 2 g, 2 g + 1 in buffer g of buf0..buf3).
template <int KIND, int NB>
__device__ __forceinline__ void wide_stage(const f32x16_t (&acc)[NB], int b0, int b1, uint16_t* buf0, uint16_t* buf1,
                                           uint16_t* buf2, uint16_t* buf3, int wv, int lane) {
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < b0 || b >= b1) continue;  // (static after unrolling)
    if constexpr (KIND == kUp) {
      uint16_t* buf = b < 4 ? buf0 : buf1;
      const int rl = 32 * (b & 3) + lr;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = silu_f(acc[b][4 * q + r]) * acc[b][4 * (q + 2) + r];
        const int c = 2 * wv + q;  // h columns 16 wv + 8 q .. + 7 of the tile
        *reinterpret_cast<uint2*>(buf + rl * 128 + ((c ^ (rl & 15)) * 8) + 4 * lh) =
            make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
      }
    } else {
      uint16_t* buf = b < 2 ? buf0 : b < 4 ? buf1 : b < 6 ? buf2 : buf3;
      const int rl = 32 * (b & 1) + lr;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = 4 * wv + k;  // columns 32 wv + 8 k .. + 7 of the tile
        *reinterpret_cast<uint2*>(buf + rl * 256 + ((c ^ (rl & 31)) * 8) + 4 * lh) =
            make_uint2(pack_bf16x2(acc[b][4 * k], acc[b][4 * k + 1]),
                       pack_bf16x2(acc[b][4 * k + 2], acc[b][4 * k + 3]));
      }
    }
  }
}

// One staged y piece (down): 16 bytes to column col of row phys, or - the
// down projection's scatter - the combine's value of a single-row token,
// round(fmaf(w, bf16(y), 0)), to its output row.
__device__ __forceinline__ void wide_store_y(const GemmArgs& p, const Tile& tl, uint16_t* out, int phys, int col,
                                             const uint4& v) {
  float sw = 0.f;
  const int st = p.sc.out != nullptr && !tl.shared ? scatter_token(p.sc, phys, sw) : -1;
  if (st < 0) {
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                reinterpret_cast<u32x4_t*>(out + size_t(phys) * p.n_out + col));
  } else {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    uint32_t o4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o4[e] = pack_bf16x2(fmaf(sw, __uint_as_float(w4[e] << 16), 0.f),
                          fmaf(sw, __uint_as_float(w4[e] & 0xffff0000u), 0.f));
    *reinterpret_cast<uint4*>(p.sc.out + size_t(st) * p.n_out + col) = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
}

// Stores of staged blocks [b0, b1) of tile tl (rows rm), from the buffers of
// wide_stage: up, instruction u = (16-row group u / 4, 32-column block u % 4)
// of the blocks, lane l takes row 16 (u / 4) + l / 4, piece 4 (u % 4) + l % 4;
// down, wave wv takes rows 8 wv .. + 7 of each 64-row buffer, two per
// instruction (lane l: piece l % 32).
template <int KIND>
__device__ __forceinline__ void wide_store(const GemmArgs& p, const Tile& tl, const int* rm, int b0, int b1,
                                           uint16_t* buf0, uint16_t* buf1, uint16_t* buf2, uint16_t* buf3, int wv,
                                           int lane) {
  const int lr = lane & 31, lh = lane >> 5;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  if constexpr (KIND == kUp) {
    const bool oblk = p.out_blk;
    for (int u = 8 * b0 + wv; u < 8 * b1; u += 8) {  // 8 instructions per 32-row block
      const int row = 16 * (u >> 2) + (lane >> 2);
      const int piece = 4 * (u & 3) + (lane & 3);
      const int phys = rm[row];
      if (phys >= 0) {
        const int rl = row & 127;
        const uint16_t* buf = row < 128 ? buf0 : buf1;
        const uint4 v = *reinterpret_cast<const uint4*>(buf + rl * 128 + ((piece ^ (rl & 15)) * 8));
        __builtin_nontemporal_store(
            u32x4_t{v.x, v.y, v.z, v.w},
            reinterpret_cast<u32x4_t*>(out + act_off(phys, tl.nt * 128 + 8 * piece, p.n_out, oblk)));
      }
    }
  } else {
    for (int g = b0 / 2; g < b1 / 2; ++g) {  // 64-row buffers
      const uint16_t* buf = g == 0 ? buf0 : g == 1 ? buf1 : g == 2 ? buf2 : buf3;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 8 * wv + 2 * i + lh;
        const int phys = rm[64 * g + rl];
        if (phys >= 0) {
          const uint4 v = *reinterpret_cast<const uint4*>(buf + rl * 256 + ((lr ^ (rl & 31)) * 8));
          wide_store_y(p, tl, out, phys, tl.nt * 256 + 8 * lr, v);
        }
      }
    }
  }
}


// Stages [s_begin, s_end) (64-deep, an even count, at least 4) of one wide
// tile with NB active 32-row activation blocks. part == nullptr: the range is
// the whole tile, run the epilogue; else leave the fp32 accumulators in part
// for ffn_wide_fixup_kernel.
template <int KIND, bool PACKED, int NB>
__device__ __forceinline__ void wide_tile(const GemmArgs& p, const Tile& tl, const int* rm, const int* ar,
                                           uint16_t* const (&X)[2], int s_begin, int s_end, float* __restrict__ part) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int last = s_end - 1;
  const int nchunks = p.K / kKC;
  constexpr int XL = NB / 2;  // activation loads per wave per stage (8 rows x 128 bytes each)

  const uint16_t* W = static_cast<const uint16_t*>(pick(tl.shared, p.sh_w, p.w));
  const int ntp = 2 * tl.nt + (wv >> 2);
  const int pw = wv & 3;
  __amdgpu_buffer_rsrc_t wr;
  uint32_t wo;
  if constexpr (PACKED) {
    wr = buf_rsrc(W + size_t(tl.we) * p.n_tiles_n * nchunks * 4 * 8 * kWave * 8);
    wo = uint32_t(((ntp * nchunks * 4 + pw) * 8 * kWave + lane) * 16);
  } else {
    wr = buf_rsrc(W + size_t(tl.we) * p.n_w_rows * p.K);
    int row;
    if (KIND == kUp) {
      const int hc = ntp * 64 + 16 * pw + (lr & 15);
      row = lr < 16 ? hc : p.n_out + hc;
    } else {
      row = ntp * 128 + 32 * pw + lr;
    }
    wo = uint32_t(row * p.K + 32 * lh) * 2u;
  }
  auto wsoff = [&](int s, int j) -> uint32_t {
    if constexpr (PACKED) return uint32_t(((s >> 1) * 4 * 8 * kWave + ((s & 1) * 4 + j) * kWave) * 16);
    else return uint32_t(64 * s + 8 * j) * 2u;
  };

  // activations: load q of this wave covers tile rows 8 (8 q + wv) .. + 7
  const uint16_t* A = static_cast<const uint16_t*>(pick(tl.shared, p.sh_a, p.a));
  const bool ablk = pick(tl.shared, p.sh_a_blk, p.a_blk);
  const uint32_t xstep = ablk ? 1024u * 2u : uint32_t(kAK) * 2u;
  const bool gat = p.a_rows != nullptr && !tl.shared;
  const int* amap = gat ? ar : rm;
  const int phys0 = amap[0];
  const size_t xbase = gat ? 0 : ablk ? blk_row_base(phys0, p.K) : size_t(phys0) * p.K;
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(A + xbase);
  uint32_t xoff[XL];
  int xlds[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int r = 8 * (kWideWaves * q + wv) + (lane >> 3);
    const int c = lane & 7;
    const int phys = amap[r];
    const int pr = phys >= 0 ? phys : phys0;
    xoff[q] = uint32_t((ablk ? blk_row_base(pr, p.K) + size_t(c >> 2) * 512 + (c & 3) * 8 : size_t(pr) * p.K + c * 8) -
                       xbase) * 2u;
    xlds[q] = r * kAK + ((c ^ ((r >> 1) & 7)) * 8);
  }
  const int fsw = (lr >> 1) & 7;
  int foff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) foff[j] = lr * kAK + (((4 * lh + j) ^ fsw) * 8);

  f32x16_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  bf16x8_t wreg[2][4];     // [stage slot][step]
  u32x4_t xs[2][XL];       // activation staging [stage slot][load]
  bf16x8_t fr[NB];

#define MOE_W8_LOAD(SLOT_, S_, J_)                                                                          \
  wreg[SLOT_][J_] = __builtin_bit_cast(                                                                     \
      bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(wr, wo, __builtin_amdgcn_readfirstlane(wsoff(S_, J_)), 0));
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0);
#define MOE_MFMA1(SLOT_, J_, B_) \
  acc[B_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[SLOT_][J_], fr[B_], acc[B_], 0, 0, 0);
  // as the 4-wave tile's stage: step j < 3 issues its MFMAs with one fragment
  // read of the next step after each (step 0 also this wave's activation loads
  // of stage s + 2); step 3 writes the staged activations of stage s + 1, holds
  // the barrier, then reads the next stage's first fragments; every step ends
  // with the weight load of stage s + 2, step j
#define MOE_W8_STEP(J_, KT_, j_)                                                                            \
  {                                                                                                         \
    MOE_FENCE()                                                                                             \
    if constexpr ((j_) < 3) {                                                                               \
      const uint32_t xo_ = __builtin_amdgcn_readfirstlane(uint32_t(min((KT_) + 2, last)) * xstep);          \
      _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                      \
        MOE_MFMA1(J_, j_, b)                                                                                \
        MOE_FENCE()                                                                                         \
        fr[b] = *reinterpret_cast<const bf16x8_t*>(X[J_] + b * 32 * kAK + foff[(j_) + 1]);                   \
        if constexpr ((j_) == 0)                                                                            \
          if (b < XL) xs[J_][b < XL ? b : 0] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[b < XL ? b : 0], xo_, 0); \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
    } else {                                                                                                \
      _Pragma("unroll") for (int b = 0; b < NB / 2; ++b) {                                                  \
        MOE_MFMA1(J_, 3, b)                                                                                 \
        MOE_FENCE()                                                                                         \
        *reinterpret_cast<u32x4_t*>(X[(J_) ^ 1] + xlds[b]) = xs[(J_) ^ 1][b];                               \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                                                               \
      __builtin_amdgcn_s_barrier();                                                                         \
      MOE_FENCE()                                                                                           \
      _Pragma("unroll") for (int b = NB / 2; b < NB; ++b) {                                                 \
        MOE_MFMA1(J_, 3, b)                                                                                 \
        MOE_FENCE()                                                                                         \
        fr[2 * b - NB] = *reinterpret_cast<const bf16x8_t*>(X[(J_) ^ 1] + (2 * b - NB) * 32 * kAK + foff[0]);    \
        fr[2 * b - NB + 1] =                                                                                \
            *reinterpret_cast<const bf16x8_t*>(X[(J_) ^ 1] + (2 * b - NB + 1) * 32 * kAK + foff[0]);         \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
    }                                                                                                       \
    MOE_W8_LOAD(J_, min((KT_) + 2, last), j_)                                                               \
  }
#define MOE_W8_STAGE(J_, KT_) \
  MOE_W8_STEP(J_, KT_, 0) MOE_W8_STEP(J_, KT_, 1) MOE_W8_STEP(J_, KT_, 2) MOE_W8_STEP(J_, KT_, 3)

#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t xo = __builtin_amdgcn_readfirstlane(uint32_t(s_begin + h) * xstep);
#pragma unroll
    for (int q = 0; q < XL; ++q) xs[h][q] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[q], xo, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) MOE_W8_LOAD(h, s_begin + h, j)
  }
#pragma unroll
  for (int q = 0; q < XL; ++q) *reinterpret_cast<u32x4_t*>(X[0] + xlds[q]) = xs[0][q];
  MOE_FENCE()
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  MOE_FENCE()
#pragma unroll
  for (int b = 0; b < NB; ++b) fr[b] = *reinterpret_cast<const bf16x8_t*>(X[0] + b * 32 * kAK + foff[0]);

  for (int kt = s_begin; kt < s_end; kt += 2) {
    MOE_W8_STAGE(0, kt)
    MOE_W8_STAGE(1, kt + 1)
  }
#undef MOE_W8_STAGE
#undef MOE_W8_STEP
#undef MOE_MFMA1
#undef MOE_FENCE
#undef MOE_W8_LOAD
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();

  if (part == nullptr) {
    if constexpr (KIND == kUp) {  // the whole tile in X[0] (rows 0-127) and X[1]
      wide_stage<KIND, NB>(acc, 0, NB, X[0], X[1], X[0], X[1], wv, lane);
      __syncthreads();
      wide_store<KIND>(p, tl, rm, 0, NB, X[0], X[1], X[0], X[1], wv, lane);
    } else {  // rounds of 64 rows in X[0], X[1] alternately (a buffer is
              // rewritten two rounds later, after a barrier that every wave
              // passes only after its reads of it)
#pragma unroll
      for (int rd = 0; rd < NB / 2; ++rd) {
        wide_stage<KIND, NB>(acc, 2 * rd, 2 * rd + 2, X[0], X[1], X[0], X[1], wv, lane);
        __syncthreads();
        wide_store<KIND>(p, tl, rm, 2 * rd, 2 * rd + 2, X[0], X[1], X[0], X[1], wv, lane);
      }
    }
  } else {
    // partial of wave w at [w / 2][w % 2]: the fixup's wave w' (4 waves) sums
    // blocks 0 and 1 of slot w', those of waves 2 w' and 2 w' + 1
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; v += 4)
        *reinterpret_cast<float4*>(part + wide_part_idx(wv >> 1, wv & 1, b, v / 4, lane)) =
            make_float4(acc[b][v], acc[b][v + 1], acc[b][v + 2], acc[b][v + 3]);
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
__global__ __launch_bounds__(kWideThreads, 1) void ffn_wide_kernel(GemmArgs p, float* __restrict__ parts) {
  __shared__ Sched sh;
  __shared__ __attribute__((aligned(1024))) uint16_t x0[kAStage], x1[kAStage];
  uint16_t* const X[2] = {x0, x1};
  const int ntn = KIND == kUp ? p.n_out / 128 : p.n_out / 256;
  const int n_tiles = build_schedule<kWideThreads>(p, kWM, ntn, true, sh);
  const int nch = p.K / kKC;
  constexpr int SPC = kKC / kAK;
  const WideSplit ws = wide_split(n_tiles, nch);
  const int slot = int(blockIdx.x % kXcds) * (kWideGrid / kXcds) + int(blockIdx.x / kXcds);
  int* meta = wide_meta(parts);
  if (blockIdx.x == 0 && threadIdx.x == 0) {  // for the fix-up
    meta[0] = ws.S > 1 ? ws.rem : 0;
    meta[1] = ws.S;
  }
  // rec: the fix-up's record of the tile (first range of a split tile), else nullptr
  auto run = [&](int t, int c_begin, int c_end, float* part, int* rec) __attribute__((always_inline)) {
    const Tile tl = decode_tile_wide(p, kWM, ntn, sh, t);
    build_rowmap<kWideThreads>(p, tl, kWM, sh, true);
    if (rec != nullptr) {  // uniform
      if (threadIdx.x == 0) {
        rec[0] = tl.nt;
        rec[1] = tl.shared;
        rec[2] = tl.nrows;
      }
      for (int i = threadIdx.x; i < tl.nrows; i += kWideThreads) rec[8 + i] = sh.rowmap[i];
    }
    const int sb = c_begin * SPC, se = c_end * SPC;
    switch ((tl.nrows + 63) / 64) {
      case 1: wide_tile<KIND, PACKED, 2>(p, tl, sh.rowmap, sh.arow, X, sb, se, part); break;
      case 2: wide_tile<KIND, PACKED, 4>(p, tl, sh.rowmap, sh.arow, X, sb, se, part); break;
      case 3: wide_tile<KIND, PACKED, 6>(p, tl, sh.rowmap, sh.arow, X, sb, se, part); break;
      default: wide_tile<KIND, PACKED, 8>(p, tl, sh.rowmap, sh.arow, X, sb, se, part); break;
    }
    __syncthreads();
  };
  for (int t = slot; t < ws.full; t += kWideGrid) run(t, 0, nch, nullptr, nullptr);
  const int u = int(blockIdx.x);
  if (ws.rem && u < ws.rem * ws.S) {
    const int i = u / ws.S, k = u % ws.S;
    if (ws.S == 1) {
      run(ws.full + i, 0, nch, nullptr, nullptr);
    } else {
      run(ws.full + i, k * nch / ws.S, (k + 1) * nch / ws.S, parts + size_t(u) * kWidePart,
          k == 0 ? meta + kWideMetaRecs + i * kWideRec : nullptr);
    }
  }
}

// Finishes the split wide tiles: block (i, b) sums the S partials of split
// tile i for activation block b in split order and runs its epilogue. The
// tile (its N tile, rows and physical rows) comes from the record its first
// range left, so a block with nothing to do ends after two loads.
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_wide_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int* meta = wide_meta(const_cast<float*>(parts));
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= __builtin_amdgcn_readfirstlane(meta[0])) return;  // uniform: not a split tile
  const int S = min(max(__builtin_amdgcn_readfirstlane(meta[1]), 1), kWideGrid);
  const int* rec = meta + kWideMetaRecs + i * kWideRec;
  Tile tl{};
  tl.nt = __builtin_amdgcn_readfirstlane(rec[0]);
  tl.shared = __builtin_amdgcn_readfirstlane(rec[1]) != 0;
  tl.nrows = min(max(__builtin_amdgcn_readfirstlane(rec[2]), 0), kWM);
  if (b * 32 >= tl.nrows) return;  // uniform: no rows in this block
  for (int r = tid; r < kWM; r += kGemmThreads) sh.rowmap[r] = r < tl.nrows ? rec[8 + r] : -1;
  __syncthreads();
  // the S partials of each accumulator tile in split order, four in flight at a time
  f32x16_t acc[2];
  sum_partials(
      acc, 0, S - 1, [&](int k) -> const float* { return parts + size_t(i * S + k) * kWidePart; },
      [&](int a, int q) { return wide_part_idx(wv, a, b, q, lane); });
  // the partials of this wave's block a are those of main-kernel wave 2 wv + a
  wide_epilogue_block<KIND>(p, tl, sh, b, acc[0], 2 * wv, lr, lh);
  wide_epilogue_block<KIND>(p, tl, sh, b, acc[1], 2 * wv + 1, lr, lh);
}

}  // namespace

moe_status_t launch_wide(const GemmArgs& p, int kind, float* parts, hipStream_t stream) {
  const dim3 grid(kWideGrid), block(kWideThreads), fblock(kGemmThreads);
  if (kind == kUp) {
    if (p.packed) hipLaunchKernelGGL((ffn_wide_kernel<kUp, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_wide_kernel<kUp, false>), grid, block, 0, stream, p, parts);
  } else {
    if (p.packed) hipLaunchKernelGGL((ffn_wide_kernel<kDown, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_wide_kernel<kDown, false>), grid, block, 0, stream, p, parts);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 wfix(kWideGrid, 8);
  if (kind == kUp) hipLaunchKernelGGL((ffn_wide_fixup_kernel<kUp>), wfix, fblock, 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_wide_fixup_kernel<kDown>), wfix, fblock, 0, stream, p, parts);
  return launch_status();
}

}  // namespace moe
