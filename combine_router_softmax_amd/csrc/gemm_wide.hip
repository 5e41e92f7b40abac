// Wide-tile grouped-GEMM kernel (prefill-shaped groups); see the kernel comment.
#include "gemm_common.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ wide-tile kernel
// Groups with many rows (prefill, and decode with few experts per GPU) are
// compute-heavy: a weight block is used by hundreds of rows. Tile = 256
// weight rows x 256 activation rows for a workgroup of 4 waves, one wave per
// SIMD; wave w owns 64 weight rows (two 32-row blocks of the packed weight
// order: up, the gate rows and the matching up rows of 32 h columns, so the
// SwiGLU pairs meet in one lane) against all 256 activation rows, a 64 x 256
// fp32 accumulator block (2 x 8 MFMA 32x32 tiles, 256 accumulator registers).
//
// What bounds this kernel on MI355X is the rate at which each compute unit
// gets operands from L2 and beyond: bytes in flight per CU against the latency
// of L2 misses (the 32 CUs of an XCD share operand slabs, but each wave still
// waits out a miss's full latency). So:
//  - the weights, private to a wave, go straight from memory into a
//    two-stage register ring (buffer loads, 1 KiB per wave instruction in the
//    packed order, each lane's 16 bytes exactly its MFMA operand), with no LDS
//    round trip;
//  - the activations, read by all 4 waves, are loaded two 64-deep stages
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

// Epilogue of one 32-row activation block b of a wide tile from the wave's two
// accumulator tiles: weight block a of wave wv is packed block 2 nt + wv / 2,
// wave slot 2 (wv % 2) + a (up: the gate rows 0-15 and up rows 16-31 of 16 h
// columns; down: 32 output columns).
template <int KIND>
__device__ __forceinline__ void wide_epilogue_block(const GemmArgs& p, const Tile& tl, const Sched& sh, int b,
                                                    const f32x16_t& a0, const f32x16_t& a1, int wv, int lr, int lh) {
  const int phys = sh.rowmap[32 * b + lr];
  if (phys < 0) return;
  uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
  const bool oblk = p.out_blk;
  uint16_t* orow = out + act_off(phys, 0, p.n_out, oblk);
  const int ntp = 2 * tl.nt + (wv >> 1);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const f32x16_t& ac = a ? a1 : a0;
    const int pw = 2 * (wv & 1) + a;
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
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = ntp * 128 + 32 * pw + 8 * q + 4 * lh;
        *reinterpret_cast<uint2*>(orow + (oblk ? size_t(col >> 5) * 512 + (col & 31) : size_t(col))) =
            make_uint2(pack_bf16x2(ac[4 * q], ac[4 * q + 1]), pack_bf16x2(ac[4 * q + 2], ac[4 * q + 3]));
      }
    }
  }
}

// Stages [s_begin, s_end) (64-deep, an even count, at least 4) of one wide
// tile. part == nullptr: the range is the whole tile, run the epilogue; else
// leave the fp32 accumulators in part for ffn_wide_fixup_kernel.
template <int KIND, bool PACKED, int NB>
__device__ __forceinline__ void wide_tile(const GemmArgs& p, const Tile& tl, const Sched& sh, uint16_t* const (&X)[2],
                                          int s_begin, int s_end, float* __restrict__ part) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int last = s_end - 1;
  const int nchunks = p.K / kKC;
  constexpr int XL = NB;  // activation loads per wave per stage (8 rows x 128 bytes each)

  // ---- weights: buffer loads from the expert's base; lane offset per block a
  const uint16_t* W = static_cast<const uint16_t*>(pick(tl.shared, p.sh_w, p.w));
  const int ntp = 2 * tl.nt + (wv >> 1);
  __amdgpu_buffer_rsrc_t wr;
  uint32_t wo[2];
  if constexpr (PACKED) {
    wr = buf_rsrc(W + size_t(tl.we) * p.n_tiles_n * nchunks * 4 * 8 * kWave * 8);
#pragma unroll
    for (int a = 0; a < 2; ++a)
      wo[a] = uint32_t(((ntp * nchunks * 4 + 2 * (wv & 1) + a) * 8 * kWave + lane) * 16);
  } else {
    wr = buf_rsrc(W + size_t(tl.we) * p.n_w_rows * p.K);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int pw = 2 * (wv & 1) + a;
      int row;
      if (KIND == kUp) {
        const int hc = ntp * 64 + 16 * pw + (lr & 15);
        row = lr < 16 ? hc : p.n_out + hc;
      } else {
        row = ntp * 128 + 32 * pw + lr;
      }
      wo[a] = uint32_t(row * p.K + 32 * lh) * 2u;
    }
  }
  // uniform byte offset of step j of stage s
  auto wsoff = [&](int s, int j) -> uint32_t {
    if constexpr (PACKED) return uint32_t(((s >> 1) * 4 * 8 * kWave + ((s & 1) * 4 + j) * kWave) * 16);
    else return uint32_t(64 * s + 8 * j) * 2u;
  };

  // ---- activations: load q of this wave covers tile rows 8 (4 q + wv) .. + 7
  const uint16_t* A = static_cast<const uint16_t*>(pick(tl.shared, p.sh_a, p.a));
  const bool ablk = pick(tl.shared, p.sh_a_blk, p.a_blk);
  const uint32_t xstep = ablk ? 1024u * 2u : uint32_t(kAK) * 2u;  // bytes from one stage of a row to the next
  const bool gat = p.a_rows != nullptr && !tl.shared;
  const int* amap = gat ? sh.arow : sh.rowmap;
  const int phys0 = amap[0];
  const size_t xbase = gat ? 0 : ablk ? blk_row_base(phys0, p.K) : size_t(phys0) * p.K;
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(A + xbase);
  uint32_t xoff[XL];
  int xlds[XL];  // LDS element offset this lane writes for load q
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int r = 8 * (4 * q + wv) + (lane >> 3);
    const int c = lane & 7;  // this lane fetches piece c of row r
    const int phys = amap[r];
    const int pr = phys >= 0 ? phys : phys0;  // rows past the tile feed only discarded columns
    xoff[q] = uint32_t((ablk ? blk_row_base(pr, p.K) + size_t(c >> 2) * 512 + (c & 3) * 8 : size_t(pr) * p.K + c * 8) -
                       xbase) * 2u;
    xlds[q] = r * kAK + ((c ^ ((r >> 1) & 7)) * 8);
  }
  // fragment of step j: row lr of each block, piece 4 lh + j, swizzled
  const int fsw = (lr >> 1) & 7;
  int foff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) foff[j] = lr * kAK + (((4 * lh + j) ^ fsw) * 8);

  f32x16_t acc[2][NB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  bf16x8_t wreg[2][2][4];  // [stage slot][a][step]
  u32x4_t xs[2][XL];       // activation staging [stage slot][load]
  bf16x8_t fr[2][NB];      // fragment sets (step parity)

#define MOE_W_LOAD(SLOT_, S_, J_)                                                                           \
  _Pragma("unroll") for (int a = 0; a < 2; ++a)                                                             \
    wreg[SLOT_][a][J_] = __builtin_bit_cast(                                                                \
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(wr, wo[a], __builtin_amdgcn_readfirstlane(wsoff(S_, J_)), 0));
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0);
  // MFMA pair (both weight blocks) of activation block B_ in step J_
#define MOE_MFMA2(SLOT_, J_, B_)                                                                            \
  acc[0][B_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[SLOT_][0][J_], fr[(J_) & 1][B_], acc[0][B_], 0, 0, 0); \
  acc[1][B_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[SLOT_][1][J_], fr[(J_) & 1][B_], acc[1][B_], 0, 0, 0);
  // one stage s (J = (s - s_begin) % 2: LDS buffer, weight slot, staging
  // slot). Step j issues its MFMA pairs with, between them, one fragment read
  // of the next step each (step 0 also one activation load of stage s + 2
  // each), then the weights of stage s + 2, step j. Step 3 writes the staged
  // activations of stage s + 1 into the other LDS buffer between its first
  // MFMA pairs, then holds the barrier that publishes them and reads the next
  // stage's first fragments between its last pairs. (The fences keep this
  // order; loads retire in order and the compiler counts every wait itself.)
#define MOE_WIDE_STEP(J_, KT_, j_)                                                                          \
  {                                                                                                         \
    MOE_FENCE()                                                                                             \
    if constexpr ((j_) < 3) {                                                                               \
      const uint32_t xo_ = __builtin_amdgcn_readfirstlane(uint32_t(min((KT_) + 2, last)) * xstep);          \
      _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                      \
        MOE_MFMA2(J_, j_, b)                                                                                \
        MOE_FENCE()                                                                                         \
        fr[((j_) + 1) & 1][b] = *reinterpret_cast<const bf16x8_t*>(X[J_] + b * 32 * kAK + foff[(j_) + 1]);   \
        if constexpr ((j_) == 0) xs[J_][b] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[b], xo_, 0);    \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
    } else {                                                                                                \
      _Pragma("unroll") for (int b = 0; b < NB / 2; ++b) {                                                  \
        MOE_MFMA2(J_, 3, b)                                                                                 \
        MOE_FENCE()                                                                                         \
        *reinterpret_cast<u32x4_t*>(X[(J_) ^ 1] + xlds[2 * b]) = xs[(J_) ^ 1][2 * b];                       \
        *reinterpret_cast<u32x4_t*>(X[(J_) ^ 1] + xlds[2 * b + 1]) = xs[(J_) ^ 1][2 * b + 1];               \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                                                               \
      __builtin_amdgcn_s_barrier();                                                                         \
      MOE_FENCE()                                                                                           \
      _Pragma("unroll") for (int b = NB / 2; b < NB; ++b) {                                                 \
        MOE_MFMA2(J_, 3, b)                                                                                 \
        MOE_FENCE()                                                                                         \
        fr[0][2 * b - NB] = *reinterpret_cast<const bf16x8_t*>(X[(J_) ^ 1] + (2 * b - NB) * 32 * kAK + foff[0]); \
        fr[0][2 * b - NB + 1] =                                                                             \
            *reinterpret_cast<const bf16x8_t*>(X[(J_) ^ 1] + (2 * b - NB + 1) * 32 * kAK + foff[0]);         \
        MOE_FENCE()                                                                                         \
      }                                                                                                     \
    }                                                                                                       \
    MOE_W_LOAD(J_, min((KT_) + 2, last), j_)                                                                \
  }
#define MOE_WIDE_STAGE(J_, KT_)                                                                             \
  MOE_WIDE_STEP(J_, KT_, 0) MOE_WIDE_STEP(J_, KT_, 1) MOE_WIDE_STEP(J_, KT_, 2) MOE_WIDE_STEP(J_, KT_, 3)

  // prologue: the activations and weights of stages 0 and 1 in the
  // steady-state order; stage 0's activations go to LDS buffer 0
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t xo = __builtin_amdgcn_readfirstlane(uint32_t(s_begin + h) * xstep);
#pragma unroll
    for (int q = 0; q < XL; ++q) xs[h][q] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[q], xo, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) MOE_W_LOAD(h, s_begin + h, j)
  }
#pragma unroll
  for (int q = 0; q < XL; ++q) *reinterpret_cast<u32x4_t*>(X[0] + xlds[q]) = xs[0][q];
  MOE_FENCE()
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  MOE_FENCE()
#pragma unroll
  for (int b = 0; b < NB; ++b) fr[0][b] = *reinterpret_cast<const bf16x8_t*>(X[0] + b * 32 * kAK + foff[0]);

  for (int kt = s_begin; kt < s_end; kt += 2) {
    MOE_WIDE_STAGE(0, kt)
    MOE_WIDE_STAGE(1, kt + 1)
  }
#undef MOE_WIDE_STAGE
#undef MOE_WIDE_STEP
#undef MOE_MFMA2
#undef MOE_FENCE
#undef MOE_W_LOAD
  // the prefetches past the range's end are drained before the registers and
  // LDS are reused; the next tile rewrites the buffers only after a barrier
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
  // the ring buffers are separate LDS objects and every access names one
  // statically, so the compiler can tell the fragment reads from the buffers
  // still being filled
  __shared__ __attribute__((aligned(1024))) uint16_t x0[kAStage], x1[kAStage];
  uint16_t* const X[2] = {x0, x1};
  const int ntn = KIND == kUp ? p.n_out / 128 : p.n_out / 256;
  const int n_tiles = build_schedule(p, kWM, ntn, true, sh);
  const int nch = p.K / kKC;  // 128-deep chunks per tile
  constexpr int SPC = kKC / kAK;  // stages per chunk
  const WideSplit ws = wide_split(n_tiles, nch);
  const int slot = int(blockIdx.x % kXcds) * (kWideGrid / kXcds) + int(blockIdx.x / kXcds);
  auto run = [&](int t, int c_begin, int c_end, float* part) __attribute__((always_inline)) {
    const Tile tl = decode_tile<true>(p, kWM, ntn, sh, t);
    build_rowmap(p, tl, kWM, sh, true);
    const int sb = c_begin * SPC, se = c_end * SPC;
    switch ((tl.nrows + 63) / 64) {
      case 1: wide_tile<KIND, PACKED, 2>(p, tl, sh, X, sb, se, part); break;
      case 2: wide_tile<KIND, PACKED, 4>(p, tl, sh, X, sb, se, part); break;
      case 3: wide_tile<KIND, PACKED, 6>(p, tl, sh, X, sb, se, part); break;
      default: wide_tile<KIND, PACKED, 8>(p, tl, sh, X, sb, se, part); break;
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

}  // namespace

moe_status_t launch_wide(const GemmArgs& p, int kind, float* parts, hipStream_t stream) {
  const dim3 grid(kWideGrid), block(kGemmThreads);
  if (kind == kUp) {
    if (p.packed) hipLaunchKernelGGL((ffn_wide_kernel<kUp, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_wide_kernel<kUp, false>), grid, block, 0, stream, p, parts);
  } else {
    if (p.packed) hipLaunchKernelGGL((ffn_wide_kernel<kDown, true>), grid, block, 0, stream, p, parts);
    else hipLaunchKernelGGL((ffn_wide_kernel<kDown, false>), grid, block, 0, stream, p, parts);
  }
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 wfix(kWideGrid, 8);
  if (kind == kUp) hipLaunchKernelGGL((ffn_wide_fixup_kernel<kUp>), wfix, block, 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_wide_fixup_kernel<kDown>), wfix, block, 0, stream, p, parts);
  return launch_status();
}

}  // namespace moe
