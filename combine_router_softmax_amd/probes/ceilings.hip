// Measured ceilings of one MI355X, the numbers the kernels' rooflines are read
// against: matrix-core peak loops (bf16 32x32x16 and fp8 32x32x64), LDS read
// bandwidth, vector-load bandwidth from L2, and a read-only HBM stream, each
// at one and at two waves per SIMD (one workgroup per compute unit; rates from
// event times). A standalone program (not part of the
// library); bench.py --ceilings runs it and prints its JSON line.
//
// Every kernel works on its own registers or on buffers it indexes with a
// power-of-two mask, so every access stays inside the allocation; each
// workgroup's thread 0 records the shader clocks its loop took.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kLdsVec = 4096;  // 64 KiB of LDS as 16-byte vectors

template <int ITERS>
__global__ __launch_bounds__(512) void lds_read(u32x4* out, long long* cyc) {
  __shared__ u32x4 buf[kLdsVec];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsVec; i += blockDim.x) buf[i] = u32x4{uint32_t(i), 1u, 2u, 3u};
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  u32x4 acc = {0, 0, 0, 0};
  const long long t0 = clock64();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= buf[((it * 8 + u) * 64 + wv * 512 + lane) & (kLdsVec - 1)];
  }
  const long long t1 = clock64();
  out[blockIdx.x * blockDim.x + tid] = acc;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

// 16-byte loads: every workgroup sweeps [base, base + mask] (vectors), base =
// blockIdx * stride, all indices masked into the buffer
template <int ITERS>
__global__ __launch_bounds__(512) void vmem_read(const u32x4* __restrict__ src, uint64_t mask, uint64_t stride,
                                                 u32x4* out, long long* cyc) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
  u32x4 acc = {0, 0, 0, 0};
  const long long t0 = clock64();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      acc ^= src[(uint64_t(blockIdx.x) * stride + uint64_t((it * 8 + u) * nw + wv) * 64 + lane) & mask];
  }
  const long long t1 = clock64();
  out[blockIdx.x * blockDim.x + tid] = acc;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

// eight independent accumulator chains per wave
template <int ITERS>
__global__ __launch_bounds__(512) void mfma_bf16(f32x16* out, long long* cyc) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = __bf16(float(tid + i) * 1e-3f);
    b[i] = __bf16(float(i) * 2e-3f);
  }
  f32x16 c[8];
  for (int j = 0; j < 8; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = float(j * 16 + v + tid);
  const long long t0 = clock64();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  const long long t1 = clock64();
  f32x16 s = c[0];
  for (int j = 1; j < 8; ++j) s += c[j];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

template <int ITERS>
__global__ __launch_bounds__(512) void mfma_fp8(f32x16* out, long long* cyc) {
  const int tid = threadIdx.x;
  i32x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 + tid + i;  // e4m3 codes near 1
    b[i] = 0x30303030 + i;
  }
  f32x16 c[8];
  for (int j = 0; j < 8; ++j)
    for (int v = 0; v < 16; ++v) c[j][v] = float(j * 16 + v + tid);
  const long long t0 = clock64();
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], 0, 0, 0, 127, 0, 127);
  }
  const long long t1 = clock64();
  f32x16 s = c[0];
  for (int j = 1; j < 8; ++j) s += c[j];
  out[blockIdx.x * blockDim.x + tid] = s;
  if (tid == 0) cyc[blockIdx.x] = t1 - t0;
}

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int grid = cus;  // one workgroup per compute unit
  u32x4* out;
  f32x16* outf;
  long long* cyc;
  CHECK(hipMalloc(&out, sizeof(u32x4) * 512 * grid));
  CHECK(hipMalloc(&outf, sizeof(f32x16) * 512 * grid));
  CHECK(hipMalloc(&cyc, sizeof(long long) * grid));
  const uint64_t big = uint64_t(1) << 31;  // 2 GiB streamed once per launch
  u32x4* src;
  CHECK(hipMalloc(&src, big));
  CHECK(hipMemset(src, 1, big));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<long long> hc(grid);
  bool first = true;
  printf("{\"device\": \"%s\", \"compute_units\": %d, \"results\": {", prop.gcnArchName, cus);
  // units per launch (bytes or flop), kernel time, mean clocks per workgroup
  auto emit = [&](const char* name, double units, const char* unit, bool per_clk) -> int {
    float ms = 0;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
    if (hipMemcpy(hc.data(), cyc, sizeof(long long) * grid, hipMemcpyDeviceToHost) != hipSuccess) return 1;
    double s = 0;
    for (int i = 0; i < grid; ++i) s += double(hc[i]);
    const double clk = s / grid;
    // (per-clock figures use the clocks wave 0 counted over its loop; with two
    // waves per SIMD that counter does not track the kernel time, so those
    // runs report rates per nanosecond only)
    printf("%s\"%s\": {\"%s_per_s\": %.4g, \"%s_per_ns_per_cu\": %.2f", first ? "" : ", ", name, unit,
           units / (ms * 1e-3), unit, units / grid / (ms * 1e6));
    if (per_clk) printf(", \"%s_per_clk_per_cu\": %.1f, \"clock_ghz\": %.3f", unit, units / grid / clk, clk / (ms * 1e6));
    printf(", \"ms\": %.4f}", ms);
    first = false;
    return 0;
  };
#define RUN(NAME, UNITS, UNIT, KERNEL, THREADS, ...)                                      \
  do {                                                                                    \
    hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(THREADS), 0, 0, __VA_ARGS__);             \
    CHECK(hipEventRecord(e0));                                                            \
    hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(THREADS), 0, 0, __VA_ARGS__);             \
    CHECK(hipEventRecord(e1));                                                            \
    CHECK(hipEventSynchronize(e1));                                                       \
    CHECK(hipGetLastError());                                                             \
    if (emit(NAME, UNITS, UNIT, (THREADS) <= 256)) return 1;                              \
  } while (0)
  constexpr int kLdsIt = 4096, kVmIt = 2048, kMfIt = 2048;
  for (int waves : {4, 8}) {
    const int th = waves * 64;
    char name[64];
    snprintf(name, sizeof name, "mfma_bf16_32x32x16_%dw", waves);
    RUN(name, double(kMfIt) * 8 * waves * 32 * 32 * 16 * 2 * grid, "flop", mfma_bf16<kMfIt>, th, outf, cyc);
    snprintf(name, sizeof name, "mfma_fp8_32x32x64_%dw", waves);
    RUN(name, double(kMfIt) * 8 * waves * 32 * 32 * 64 * 2 * grid, "flop", mfma_fp8<kMfIt>, th, outf, cyc);
    snprintf(name, sizeof name, "lds_read_b128_%dw", waves);
    RUN(name, double(kLdsIt) * 8 * th * 16 * grid, "bytes", lds_read<kLdsIt>, th, out, cyc);
    // every workgroup rereads the same 1 MiB: L2 hits after the first pass
    snprintf(name, sizeof name, "l2_read_1MiB_%dw", waves);
    RUN(name, double(kVmIt) * 8 * th * 16 * grid, "bytes", vmem_read<kVmIt>, th, src, uint64_t((1 << 16) - 1),
        uint64_t(0), out, cyc);
    // each workgroup streams its own part of 2 GiB
    snprintf(name, sizeof name, "hbm_read_stream_%dw", waves);
    RUN(name, double(kVmIt) * 8 * th * 16 * grid, "bytes", vmem_read<kVmIt>, th, src, big / 16 - 1,
        big / 16 / grid, out, cyc);
  }
#undef RUN
  printf("}}\n");
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(outf));
  CHECK(hipFree(cyc));
  return 0;
}
