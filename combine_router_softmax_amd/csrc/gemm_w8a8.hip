// W8A8 grouped-GEMM kernel: fp8 activations x fp8 weights with block scales;
// see the kernel comment.
#include "fp8_quant.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

// ------------------------------------------------------------------ W8A8 kernel
// Perplexity, "Lower latency and higher throughput with multi-node DeepSeek
// deployment", section Quantization: weights carry one fp32 scale per 128 x
// 128 tile, activations one per 128-element vector, so along the reduction the
// scales change every 128 elements. Per 128-deep chunk c of an output
// element: out += sa[row, c] * sw[n / 128, c] * (the chunk's fp8 dot product).
// The dot product runs on v_mfma_scale_f32_32x32x64_f8f6f4 (two instructions
// per chunk, e4m3 x e4m3, hardware scales left at 1) into a temporary; the
// scaled sum into the fp32 accumulator is a vector-ALU multiply-add per
// element and chunk. (The matrix instruction's internal sum is not an exact
// fp32 sum of its 64 products - measured here up to about 3e-4 of the largest
// product - so the per-chunk promotion into fp32 registers is needed anyway,
// as the page says of its hardware.)
//
// Tiles, schedule, stream-K ranges and the fix-up follow the fp8-weight
// (W8A16) kernel: 96 activation rows x four N blocks (512 weight rows) per
// tile. The workgroup is 4 waves, one per SIMD, so each wave has 512
// registers: wave w owns weight rows 32 w .. + 31 of all four N blocks
// (sub-blocks a = 0..3), i.e. 12 accumulator tiles, two chunks of weights in
// flight (128 registers) and the staged activations, without spilling (eight
// waves at 256 registers each spilled in the loop). An up-projection pair of
// sub-blocks (a = 2 p, 2 p + 1) covers 2 x 64 h columns = one 128-column
// block of h over the four waves, so the epilogue can quantize h itself:
// h = silu(g) * u in fp32, the block's largest magnitude through LDS, then
// codes and one scale per (row, 128 columns) (the page's SiLU step with its
// 128-element max reduction). The down projection writes bf16 (the return
// path is bf16).
//
// Data path per chunk: weights straight from HBM into registers (each lane 64
// contiguous bytes of its row, packed or row-major, as the W8A16 kernel), two
// chunks ahead; the chunk's activation codes [96 rows x 128 bytes] by 16-byte
// loads into registers, two chunks ahead, then written to one of two LDS
// stages one chunk ahead (16-byte slot s of staged row r holds piece
// s ^ (r % 8), so the fragment reads of 8 neighbouring rows hit 8 different
// bank groups); scales by 4-byte loads. Only ordinary loads: LDS DMA
// (global_load_lds) was tried here with hand-counted waits and gave rows of
// stale activations now and then - its completion is not ordered with the
// loads into registers that the count assumed.
// B operand of lane (row lr, half lh) in instruction m: bytes 64 lh + 32 m ..
// + 31 of the row's chunk, the same k range the weights' lane holds in its
// bytes 32 m .. + 31 (the packed and row-major weight layouts both give lane
// half lh the chunk's bytes 64 lh .. + 63).
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kQ8Waves = 4;                  // one per SIMD
constexpr int kQ8Threads = kQ8Waves * kWave;
constexpr int kQ8NA = kF8NB;                 // N blocks (sub-blocks) per wave
constexpr int kQ8Stage = kF8BM * kKC;        // bytes per LDS stage (96 rows)
constexpr int kQ8Interleave = 6;             // whole tiles per range from which ranges interleave
constexpr int kQ8WaitLgkm0 = waitcnt_vm(63) & ~(15 << 8);  // LDS ops only

__device__ __forceinline__ float* q8_slot(float* parts, int b, int slot) {
  return parts + (size_t(b) * 2 + slot) * kF8PartFloats;
}
// [wave][sub-block a][block][quad q][lane][4 floats]: 1 KiB contiguous per wave access
__device__ __forceinline__ int q8_part_idx(int wv, int a, int b, int q, int lane) {
  return ((((wv * kQ8NA + a) * kF8MB + b) * 4 + q) * kWave + lane) * 4;
}
static_assert(kQ8Waves * kQ8NA * kF8MB * 16 * kWave <= kF8PartFloats, "a workgroup's accumulators fit a partial slot");

__device__ __forceinline__ i32x8_t q8_cat(const uint4& lo, const uint4& hi) {
  i32x8_t v;
  v[0] = int(lo.x); v[1] = int(lo.y); v[2] = int(lo.z); v[3] = int(lo.w);
  v[4] = int(hi.x); v[5] = int(hi.y); v[6] = int(hi.z); v[7] = int(hi.w);
  return v;
}

__device__ __forceinline__ f32x16_t q8_mfma(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c) {
  // formats 0 / 0: e4m3 x e4m3; scale selectors 0, scales 127 (E8M0 for 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// acc += f * t, registers 0..7 with flo and 8..15 with fhi (up: gate rows,
// up rows of the wave's 32 weight rows)
__device__ __forceinline__ void q8_fold(f32x16_t& acc, const f32x16_t& t, float flo, float fhi) {
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = fmaf(t[v], flo, acc[v]);
#pragma unroll
  for (int v = 8; v < 16; ++v) acc[v] = fmaf(t[v], fhi, acc[v]);
}

// LDS writes of every wave visible to every wave (no wait for global memory,
// so the prefetched loads stay in flight); the empty asm keeps the compiler
// from moving memory accesses across it
__device__ __forceinline__ void q8_lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kQ8WaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SwiGLU of one 32-row block of a pair of a wave's accumulators (g0: N block
// nb0, g1: nb0 + 1): h = silu(gate) * up into registers 0..7 of each; returns
// the largest |h| of the lane's row over the wave's 16 columns (both halves).
__device__ __forceinline__ float q8_swiglu(f32x16_t& g0, f32x16_t& g1) {
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      g0[4 * q + r] = silu_f(g0[4 * q + r]) * g0[4 * (q + 2) + r];
      g1[4 * q + r] = silu_f(g1[4 * q + r]) * g1[4 * (q + 2) + r];
      m = fmaxf(m, fmaxf(fabsf(g0[4 * q + r]), fabsf(g1[4 * q + r])));
    }
  return fmaxf(m, __shfl_xor(m, 32));
}

// Codes of the wave's 16 h columns of row phys (registers 0..7 of g0, g1) and,
// from one lane per row, the block's scale.
__device__ __forceinline__ void q8_store_h(const f32x16_t& g0, const f32x16_t& g1, float s, int nb0, int64_t phys,
                                           uint8_t* hq, float* hs, int I, int wq, int lh) {
  uint8_t* row = hq + size_t(phys) * I;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x16_t& g = a ? g1 : g0;
      const uint32_t w = e4m3_quant4(g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3], s);
      const int col = 64 * (nb0 + a) + 16 * wq + 8 * q + 4 * lh;
      *reinterpret_cast<uint32_t*>(row + col) = w;
    }
  if (wq == 0 && lh == 0) hs[size_t(phys) * (I / 128) + (nb0 >> 1)] = s;
}

// Tiles tl.nt .. tl.nt + n - 1 of one group and row tile, iterations
// [it_begin, it_end) of the run (as the W8A16 kernel's run).
template <int KIND, bool PACKED, int NB, bool STREAM>
__device__ __forceinline__ void q8_run(const GemmArgs& p, const Tile& tl, int n, const Sched& sh,
                                       uint8_t* __restrict__ x0, uint8_t* __restrict__ x1,
                                       float* __restrict__ red, int it_begin, int it_end,
                                       float* __restrict__ part_first, float* __restrict__ part_last) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // 0..3: the wave's 32 rows of each N block
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nchunks = __builtin_amdgcn_readfirstlane(p.K / kKC);
  it_begin = __builtin_amdgcn_readfirstlane(it_begin);
  it_end = __builtin_amdgcn_readfirstlane(it_end);
  n = __builtin_amdgcn_readfirstlane(n);
  const int last = it_end - 1;
  const int nt0 = __builtin_amdgcn_readfirstlane(kF8NB * tl.nt);
  const int nt_max = __builtin_amdgcn_readfirstlane(p.n_tiles_n - 1);
  // N block of sub-block a of the run's tile k (past the group's last block a
  // sub-block repeats it; its results are discarded)
  auto ntof = [&](int k, int a) { return min(nt0 + kF8NB * k + a, nt_max); };

  // weights (as the W8A16 kernel)
  const uint8_t* W = static_cast<const uint8_t*>(pick(tl.shared, p.sh_w, p.w));
  int wrow0;
  if (KIND == kUp) {
    const int j = 16 * wv + (lr & 15);
    wrow0 = lr < 16 ? j : p.n_out + j;
  } else {
    wrow0 = 32 * wv + lr;
  }
  __amdgpu_buffer_rsrc_t rw;
  uint32_t woff;
  if constexpr (PACKED) {
    rw = buf_rsrc(W + size_t(tl.we) * p.n_tiles_n * nchunks * 4 * 4 * kWave * 16);
    woff = uint32_t(wv * 4 * kWave + lane) * 16u;
  } else {
    rw = buf_rsrc(W + size_t(tl.we) * p.n_w_rows * p.K);
    woff = uint32_t(wrow0 * p.K + 64 * lh);
  }
  auto wsoff = [&](int k, int C, int a) -> int {
    const int nt = ntof(k, a);
    if constexpr (PACKED) return (nt * nchunks + C) * 4 * 4 * kWave * 16;
    else return nt * (KIND == kUp ? 64 : 128) * p.K + C * kKC;
  };
  // pieces 2 m and 2 m + 1 of sub-block a: the A operand of instruction m,
  // loaded straight into one 8-register tuple
  auto wpair = [&](int k, int C, int a, int m) -> i32x8_t {
    constexpr int aux = STREAM ? 2 : 0;  // non-temporal: the weights are read once
    const int so = wsoff(k, C, a);
    const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(
        rw, woff, __builtin_amdgcn_readfirstlane(so + (PACKED ? 2 * m * kWave * 16 : 2 * m * 16)), aux);
    const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(
        rw, woff, __builtin_amdgcn_readfirstlane(so + (PACKED ? (2 * m + 1) * kWave * 16 : (2 * m + 1) * 16)), aux);
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // weight scales, uniform per wave: up: gate rows of N block nt lie in 128-row
  // block nt / 2, its up rows in I / 128 + nt / 2; down: block nt
  constexpr int NSW = KIND == kUp ? 2 : 1;
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(pick(tl.shared, p.sh_s, p.s) + size_t(tl.we) * (p.n_w_rows / 128) * nchunks);
  auto wscale = [&](int k, int C, int a, int j) {
    const int nt = ntof(k, a);
    const int blk = KIND == kUp ? (j ? p.n_out / 128 + (nt >> 1) : nt >> 1) : nt;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs, 0u, __builtin_amdgcn_readfirstlane((blk * nchunks + C) * 4), 0));
  };

  // activations: codes [rows, K] bytes; staging load q of wave wv brings tile
  // rows 8 (4 q + wv) .. + 7 (lane: row + lane / 8, slot lane % 8), q < NB
  const uint8_t* A = static_cast<const uint8_t*>(pick(tl.shared, p.sh_a, p.a));
  const float* AS = pick(tl.shared, p.sh_as, p.as);
  const bool gat = p.a_rows != nullptr && !tl.shared;
  const int* amap = gat ? sh.arow : sh.rowmap;
  const int phys0 = amap[0];
  const size_t xbase = gat ? 0 : size_t(phys0) * p.K;
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(A + xbase);
  uint32_t xoff[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int r = 8 * (kQ8Waves * q + wv) + (lane >> 3);
    const int c = (lane & 7) ^ (r & 7);
    const int phys = amap[r];
    const int pr = phys >= 0 ? phys : phys0;  // rows past the tile feed only discarded columns
    xoff[q] = uint32_t(size_t(pr) * p.K + c * 16 - xbase);
  }
  u32x4_t xs[NB];  // the staged chunk between its load and its LDS write
  auto xload = [&](int C) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      xs[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[q], __builtin_amdgcn_readfirstlane(C * kKC), 0);
  };
  auto xstore = [&](uint8_t* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      *reinterpret_cast<u32x4_t*>(stage + (kQ8Waves * q + wv) * 1024 + lane * 16) = xs[q];
  };
  // activation scales [rows, K / 128]: the lane's row of each 32-row block
  const int kb = p.K / kKC;
  const __amdgpu_buffer_rsrc_t ra = buf_rsrc(AS);
  uint32_t aoff[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int phys = amap[32 * b + lr];
    aoff[b] = uint32_t(size_t(phys >= 0 ? phys : phys0) * kb * 4);
  }
  auto ascale = [&](int C, int b) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, aoff[b], __builtin_amdgcn_readfirstlane(C * 4), 0));
  };

  f32x16_t acc[kQ8NA][NB];
#pragma unroll
  for (int a = 0; a < kQ8NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  const f32x16_t zero = {};

  // Ring (every period 2): iteration I (counted from it_begin) computes from
  // LDS stage, weight set and scale set (I - it_begin) % 2. At the end of I,
  // after its last matrix instruction: the staged chunk of I + 1 (loaded at
  // the end of I - 1) goes to the other stage (all waves left it at the
  // barrier at the top of I), then the scales, the activation chunk and the
  // weights of I + 2 are requested (into I's sets). The barrier at the top of
  // I + 1 makes every wave's stage writes visible. All loads are ordinary
  // ones, so the compiler's waits before each use are exact: the weights and
  // scales have two iterations, the activations one (they mostly come from L2).
  i32x8_t w0[kQ8NA][2], w1[kQ8NA][2];  // [sub-block][instruction]
  float sw0[kQ8NA][NSW], sw1[kQ8NA][NSW];
  float sa0[NB], sa1[NB];
  int k_cur = __builtin_amdgcn_readfirstlane(it_begin / nchunks);
  int c_cur = __builtin_amdgcn_readfirstlane(it_begin - k_cur * nchunks);
  int i_ld = it_begin, k_ld = k_cur, c_ld = c_cur;
  auto adv_ld = [&]() __attribute__((always_inline)) {
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
  const int fr_row = lr * kKC;
  const int fr_x = lr & 7;
#define MOE_Q8_SCALES(SWN_, SAN_)                                                                           \
  {                                                                                                         \
    const int k_ = k_ld, c_ = c_ld;                                                                         \
    _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a)                                                       \
      _Pragma("unroll") for (int j = 0; j < NSW; ++j) SWN_[a][j] = wscale(k_, c_, a, j);                    \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) SAN_[b] = ascale(c_, b);                                 \
  }
#define MOE_Q8_WLOAD(WR_)                                                                                   \
  _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a)                                                         \
    _Pragma("unroll") for (int m = 0; m < 2; ++m) WR_[a][m] = wpair(k_ld, c_ld, a, m);
  // the chunk's matrix products and their scaled sums: pair i = (block b,
  // sub-block a) in order b, a into temporary i % 2; the scaled sum of pair
  // i - 1 is taken while pair i's instructions run
#define MOE_Q8_COMPUTE(XBUF_, WR_, SW_, SA_)                                                                \
  {                                                                                                         \
    int fx_ = fr_x;                                                                                         \
    asm volatile("" : "+v"(fx_));                                                                           \
    f32x16_t t_[2];                                                                                         \
    _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                        \
      const uint8_t* xr_ = (XBUF_) + b * 32 * kKC + fr_row;                                                 \
      const uint4 p0_ = *reinterpret_cast<const uint4*>(xr_ + (((4 * lh + 0) ^ fx_) * 16));                 \
      const uint4 p1_ = *reinterpret_cast<const uint4*>(xr_ + (((4 * lh + 1) ^ fx_) * 16));                 \
      const uint4 p2_ = *reinterpret_cast<const uint4*>(xr_ + (((4 * lh + 2) ^ fx_) * 16));                 \
      const uint4 p3_ = *reinterpret_cast<const uint4*>(xr_ + (((4 * lh + 3) ^ fx_) * 16));                 \
      const i32x8_t fb0_ = q8_cat(p0_, p1_), fb1_ = q8_cat(p2_, p3_);                                       \
      _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a) {                                                   \
        const int i_ = b * kQ8NA + a;                                                                       \
        t_[i_ & 1] = q8_mfma(WR_[a][0], fb0_, zero);                                                        \
        t_[i_ & 1] = q8_mfma(WR_[a][1], fb1_, t_[i_ & 1]);                                                  \
        if (i_ > 0) {                                                                                       \
          const int pb_ = (i_ - 1) / kQ8NA, pa_ = (i_ - 1) % kQ8NA;                                         \
          q8_fold(acc[pa_][pb_], t_[(i_ - 1) & 1], SA_[pb_] * SW_[pa_][0], SA_[pb_] * SW_[pa_][NSW - 1]);   \
        }                                                                                                   \
      }                                                                                                     \
    }                                                                                                       \
    q8_fold(acc[kQ8NA - 1][NB - 1], t_[(NB * kQ8NA - 1) & 1], SA_[NB - 1] * SW_[kQ8NA - 1][0],              \
            SA_[NB - 1] * SW_[kQ8NA - 1][NSW - 1]);                                                         \
  }
  // after iteration I_: if it ends its tile, the tile's epilogue (or partial
  // sums) and fresh accumulators
#define MOE_Q8_FINISH(I_)                                                                                   \
  {                                                                                                         \
    const int k_ = k_cur;                                                                                   \
    if (c_cur == nchunks - 1 || (I_) == last) { /* uniform */                                               \
      float* part_ = k_ == 0 ? part_first : (k_ == n - 1 ? part_last : nullptr);                            \
      if (part_ == nullptr) {                                                                               \
        if constexpr (KIND == kUp) {                                                                        \
          float m_[2][NB];                                                                                  \
          _Pragma("unroll") for (int pp = 0; pp < 2; ++pp)                                                  \
            _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                \
              m_[pp][b] = q8_swiglu(acc[2 * pp][b], acc[2 * pp + 1][b]);                                    \
              if (lh == 0) red[((pp * kF8MB + b) * kQ8Waves + wv) * 32 + lr] = m_[pp][b];                   \
            }                                                                                               \
          q8_lds_barrier();                                                                                 \
          uint8_t* hq_ = static_cast<uint8_t*>(pick(tl.shared, p.sh_out, p.out));                           \
          float* hs_ = pick(tl.shared, p.sh_out_s, p.out_s);                                                \
          _Pragma("unroll") for (int pp = 0; pp < 2; ++pp) {                                                \
            const int nb0_ = kF8NB * (tl.nt + k_) + 2 * pp;                                                 \
            _Pragma("unroll") for (int b = 0; b < NB; ++b) {                                                \
              const float* rb_ = red + (pp * kF8MB + b) * kQ8Waves * 32 + lr;                               \
              const float s_ = e4m3_block_scale(fmaxf(fmaxf(rb_[0], rb_[32]), fmaxf(rb_[64], rb_[96])));     \
              const int phys_ = sh.rowmap[32 * b + lr];                                                     \
              if (nb0_ < p.n_tiles_n && phys_ >= 0)                                                         \
                q8_store_h(acc[2 * pp][b], acc[2 * pp + 1][b], s_, nb0_, phys_, hq_, hs_, p.n_out, wv, lh); \
            }                                                                                               \
          }                                                                                                 \
        } else {                                                                                            \
          uint16_t* y_ = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));                          \
          _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a) {                                               \
            Tile ta_ = tl;                                                                                  \
            ta_.nt = kF8NB * (tl.nt + k_) + a;                                                              \
            if (ta_.nt < p.n_tiles_n) ffn_epilogue<KIND, NB>(acc[a], ta_, NB, sh, y_, p.n_out, wv, lr, lh, false, p.sc); \
          }                                                                                                 \
        }                                                                                                   \
      } else {                                                                                              \
        _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a)                                                   \
          _Pragma("unroll") for (int b = 0; b < NB; ++b)                                                    \
            _Pragma("unroll") for (int v = 0; v < 16; v += 4)                                               \
              *reinterpret_cast<float4*>(part_ + q8_part_idx(wv, a, b, v / 4, lane)) =                      \
                  make_float4(acc[a][b][v], acc[a][b][v + 1], acc[a][b][v + 2], acc[a][b][v + 3]);          \
      }                                                                                                     \
      _Pragma("unroll") for (int a = 0; a < kQ8NA; ++a)                                                     \
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
  // iteration I_ from stage XBUF_ with weights WR_ and scales SW_, SA_; the
  // chunk of I_ + 1 goes to stage XN_, the loads of I_ + 2 into WR_, SW_, SA_
#define MOE_Q8_ITER(I_, XBUF_, XN_, WR_, SW_, SA_)                                                          \
  {                                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    __builtin_amdgcn_s_waitcnt(kQ8WaitLgkm0);                                                               \
    __builtin_amdgcn_s_barrier();                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_Q8_COMPUTE(XBUF_, WR_, SW_, SA_)                                                                    \
    /* the next loads may not move up into the computation (their registers */                              \
    /* would then live beside the ones it still reads) */                                                   \
    asm volatile("" ::: "memory");                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    xstore(XN_);                                                                                            \
    adv_ld(); /* to min(I_ + 2, last): past the end a harmless repeat */                                    \
    MOE_Q8_SCALES(SW_, SA_)                                                                                 \
    xload(c_ld);                                                                                            \
    MOE_Q8_WLOAD(WR_)                                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                                      \
    MOE_Q8_FINISH(I_)                                                                                       \
  }

  MOE_Q8_SCALES(sw0, sa0)
  xload(c_ld);
  MOE_Q8_WLOAD(w0)
  xstore(x0);
  adv_ld();
  MOE_Q8_SCALES(sw1, sa1)
  xload(c_ld);
  MOE_Q8_WLOAD(w1)
  int it = it_begin;
  for (; it + 2 <= it_end; it += 2) {
    MOE_Q8_ITER(it, x0, x1, w0, sw0, sa0)
    MOE_Q8_ITER(it + 1, x1, x0, w1, sw1, sa1)
  }
  if (it < it_end) MOE_Q8_ITER(it, x0, x1, w0, sw0, sa0)
#undef MOE_Q8_ITER
#undef MOE_Q8_FINISH
#undef MOE_Q8_COMPUTE
#undef MOE_Q8_WLOAD
#undef MOE_Q8_SCALES
  // every wave has left the stages before the next run writes them
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  __builtin_amdgcn_s_barrier();
}

// Stream-K over (tile, chunk) iterations with the W8A16 kernel's tiles and ranges.
// INTERLEAVE: the instantiation for prefill-sized launches (below); decode
// launches take the other, whose code then holds no trace of it.
template <int KIND, bool PACKED, bool INTERLEAVE>
__global__ __launch_bounds__(kQ8Threads, 1) void ffn_w8a8_kernel(GemmArgs p, float* __restrict__ parts) {
  __shared__ Sched sh;
  __shared__ __attribute__((aligned(1024))) uint8_t x0[kQ8Stage], x1[kQ8Stage];
  __shared__ float red[2 * kF8MB * kQ8Waves * 32];
  const int ntn4 = (p.n_tiles_n + kF8NB - 1) / kF8NB;
  const int n_tiles = build_schedule<kQ8Threads>(p, kF8BM, ntn4, false, sh);
  const int nchunks = p.K / kKC;
  const DpSk sp = dpsk_split(n_tiles, nchunks, kF8Grid);
  if (int(blockIdx.x) >= sp.G) return;  // uniform
  const int G = sp.G;
  const int rng = xcd_range(int(blockIdx.x), G);
  int* meta = sk_meta(parts, kF8PartFloats, kF8Grid);
  sk_meta_begin(meta, sp, rng);
  // Many whole tiles per range (prefill sizes): range r takes whole tiles r,
  // r + G, r + 2G, ... instead of a contiguous run of them. An (expert, N
  // tile)'s row tiles are consecutive in the tile order, so the workgroups of
  // an XCD, which hold consecutive ranges, then stream the same weight slab
  // together and its L2 serves the repeats; with contiguous runs one
  // workgroup streamed the slab once per row tile, one after another.
  const bool inter = INTERLEAVE && sp.whole >= kQ8Interleave;
  if (inter) {  // uniform
    for (int j = 0; j < sp.whole; ++j) {
      const int t = j * G + rng;  // < G * whole <= n_tiles
      const Tile tl = decode_tile(p, kF8BM, ntn4, sh, t);
      build_rowmap<kQ8Threads>(p, tl, kF8BM, sh, true);
      switch ((tl.nrows + 31) / 32) {
        case 1: q8_run<KIND, PACKED, 1, false>(p, tl, 1, sh, x0, x1, red, 0, nchunks, nullptr, nullptr); break;
        case 2: q8_run<KIND, PACKED, 2, false>(p, tl, 1, sh, x0, x1, red, 0, nchunks, nullptr, nullptr); break;
        default: q8_run<KIND, PACKED, 3, false>(p, tl, 1, sh, x0, x1, red, 0, nchunks, nullptr, nullptr); break;
      }
      __syncthreads();  // rowmap is rewritten by the next tile
    }
  }
  // the range's whole tiles first (unless taken above), then its share of the
  // remainder
  for (int part = inter ? 1 : 0; part < 2; ++part) {
    const int64_t i0 = part == 0 ? int64_t(rng) * sp.whole * nchunks : sp.rem_base + sk_start(rng, sp.rem, G);
    const int64_t i1 = part == 0 ? min(int64_t(rng + 1) * sp.whole, int64_t(n_tiles)) * nchunks
                                 : sp.rem_base + sk_start(rng + 1, sp.rem, G);
    if (i0 >= i1) continue;  // uniform
    const int t_first = int(i0 / nchunks), t_last = int((i1 - 1) / nchunks);
    const bool rec_cut = part == 1 && sk_owns_cut(i0, i1, nchunks);  // the fix-up's record of tile t_last
    for (int t = t_first; t <= t_last;) {
      const Tile tl = decode_tile(p, kF8BM, ntn4, sh, t);
      build_rowmap<kQ8Threads>(p, tl, kF8BM, sh, true);
      const int n = tl.mtiles == 1 ? min(t_last - t + 1, ntn4 - tl.nt) : 1;
      if (rec_cut && t_last < t + n)  // uniform
        sk_write_rec<kQ8Threads>(meta, rng, t_last, t, tl, sh,
                         sk_owner(int64_t(t_last + 1) * nchunks - 1 - sp.rem_base, sp.rem, G));
      const int64_t t0 = int64_t(t) * nchunks;
      const int it_begin = int(max<int64_t>(i0 - t0, 0));
      const int it_end = int(min<int64_t>(i1 - t0, int64_t(n) * nchunks));
      const bool split_first = it_begin > 0 || (n == 1 && it_end < nchunks);
      const bool split_last = it_end < n * nchunks;
      float* part_first = split_first ? q8_slot(parts, rng, t == t_first ? 0 : 1) : nullptr;
      float* part_last = n == 1 ? part_first : (split_last ? q8_slot(parts, rng, 1) : nullptr);
      auto run = [&](auto stream_tag) __attribute__((always_inline)) {
        constexpr bool ST = decltype(stream_tag)::value;
        switch ((tl.nrows + 31) / 32) {
          case 1: q8_run<KIND, PACKED, 1, ST>(p, tl, n, sh, x0, x1, red, it_begin, it_end, part_first, part_last); break;
          case 2: q8_run<KIND, PACKED, 2, ST>(p, tl, n, sh, x0, x1, red, it_begin, it_end, part_first, part_last); break;
          default: q8_run<KIND, PACKED, 3, ST>(p, tl, n, sh, x0, x1, red, it_begin, it_end, part_first, part_last); break;
        }
      };
      if (tl.mtiles == 1) run(std::true_type{});
      else run(std::false_type{});
      __syncthreads();  // rowmap is rewritten by the next run
      t += n;
    }
  }
}

// Finishes the tiles cut by a range boundary: block (j, pr * kF8MB + b) takes
// the tile's N-block pair pr (N blocks 2 pr, 2 pr + 1 of the tile: one
// 128-column block of h for the up projection) and 32-row block b, with one
// wave per 32 weight rows of each N block (the partials of the main kernel's
// wave wv, sub-blocks 2 pr and 2 pr + 1).
template <int KIND>
__global__ __launch_bounds__(kGemmThreads) void ffn_w8a8_fixup_kernel(GemmArgs p, const float* __restrict__ parts) {
  __shared__ Sched sh;
  __shared__ float red[4 * 32];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int lr = lane & 31;
  const int lh = lane >> 5;
  const int nchunks = p.K / kKC;
  const int j = blockIdx.x, pr = blockIdx.y / kF8MB, b = blockIdx.y % kF8MB;
  // the tile and its ranges from the record range j left (no schedule rebuilt;
  // the whole-tile parts never cut a tile)
  const int* meta = sk_meta(const_cast<float*>(parts), kF8PartFloats, kF8Grid);
  SkRec r;
  if (!sk_read_rec(meta, j, kF8BM, r)) return;  // uniform: the boundary after range j is no tile's first cut
  const DpSk sp = r.sp;
  const int G = sp.G, t = r.t, b_lo = r.b_lo, b_hi = r.b_hi;
  const Tile tl = r.tl;
  const int nb0 = kF8NB * tl.nt + 2 * pr;
  if (b * 32 >= tl.nrows || nb0 >= p.n_tiles_n) return;  // uniform: no rows / no such N block
  sk_read_rows<kGemmThreads>(meta, j, kF8BM, tl.nrows, sh);
  f32x16_t acc[2];
  sum_partials(
      acc, b_lo, b_hi,
      [&](int w) -> const float* {
        const int64_t s0 = sp.rem_base + sk_start(w, sp.rem, G), s1 = sp.rem_base + sk_start(w + 1, sp.rem, G);
        return s0 < s1 ? q8_slot(const_cast<float*>(parts), w, int(s0 / nchunks) == t ? 0 : 1) : nullptr;
      },
      [&](int a, int q) { return q8_part_idx(wv, 2 * pr + a, b, q, lane); });
  const int phys = sh.rowmap[b * 32 + lr];
  if constexpr (KIND == kUp) {
    const float m = q8_swiglu(acc[0], acc[1]);
    if (lh == 0) red[wv * 32 + lr] = m;
    __syncthreads();
    const float s = e4m3_block_scale(fmaxf(fmaxf(red[lr], red[32 + lr]), fmaxf(red[64 + lr], red[96 + lr])));
    if (phys >= 0)
      q8_store_h(acc[0], acc[1], s, nb0, phys, static_cast<uint8_t*>(pick(tl.shared, p.sh_out, p.out)),
                 pick(tl.shared, p.sh_out_s, p.out_s), p.n_out, wv, lh);
  } else {
    uint16_t* out = static_cast<uint16_t*>(pick(tl.shared, p.sh_out, p.out));
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      Tile ta = tl;
      ta.nt = nb0 + a;
      if (ta.nt < p.n_tiles_n) ffn_epilogue_block<KIND>(acc[a], ta, b, sh, out, p.n_out, wv, lr, lh, false, p.sc);
    }
  }
}

}  // namespace

moe_status_t launch_w8a8(const GemmArgs& p, int kind, float* parts, hipStream_t stream) {
  const dim3 grid(kF8Grid), block(kQ8Threads);
#define MOE_Q8_LAUNCH(KIND_, PACKED_, INTER_) \
  hipLaunchKernelGGL((ffn_w8a8_kernel<KIND_, PACKED_, INTER_>), grid, block, 0, stream, p, parts)
  const bool il = p.interleave != 0;
  if (kind == kUp) {
    if (p.packed) {
      if (il) MOE_Q8_LAUNCH(kUp, true, true);
      else MOE_Q8_LAUNCH(kUp, true, false);
    } else {
      if (il) MOE_Q8_LAUNCH(kUp, false, true);
      else MOE_Q8_LAUNCH(kUp, false, false);
    }
  } else {
    if (p.packed) {
      if (il) MOE_Q8_LAUNCH(kDown, true, true);
      else MOE_Q8_LAUNCH(kDown, true, false);
    } else {
      if (il) MOE_Q8_LAUNCH(kDown, false, true);
      else MOE_Q8_LAUNCH(kDown, false, false);
    }
  }
#undef MOE_Q8_LAUNCH
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  const dim3 fix_grid(kF8Grid - 1, 2 * kF8MB);
  if (kind == kUp) hipLaunchKernelGGL((ffn_w8a8_fixup_kernel<kUp>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  else hipLaunchKernelGGL((ffn_w8a8_fixup_kernel<kDown>), fix_grid, dim3(kGemmThreads), 0, stream, p, parts);
  return launch_status();
}

}  // namespace moe
