// Shared device/host helpers of the gfx950 MoE library (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "moe.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> two RNE bf16 in one dword (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------- host checks
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(moe_dtype_t dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3: return 1;
  }
  return 0;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Compute units of the current device (cached per device; immutable data).
int device_cu_count();

// Map the result of a launch to a status.
inline moe_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// Block-wide scan of a[0..n) in LDS (kThreads threads). Each thread
// scans a contiguous run, then the run totals are scanned across the block;
// up to one wavefront of values, the first wave scans them alone with lane
// shuffles (two barriers instead of two per doubling step). kMax: inclusive
// max-scan; otherwise exclusive sum-scan with the total returned. All threads
// must call it.
template <bool kMax, int kThreads>
__device__ int block_scan_lds(int* a, int n, int* tmp /* [kThreads] */) {
  const int tid = threadIdx.x;
  if (n <= kWave) {  // uniform
    if (tid < kWave) {
      const int id = kMax ? INT_MIN : 0;
      const int v = tid < n ? a[tid] : id;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (tid >= off) incl = kMax ? max(incl, u) : incl + u;
      }
      if (tid < n) a[tid] = kMax ? incl : incl - v;
      if (tid == kWave - 1) tmp[0] = incl;
    }
    __syncthreads();
    const int total = tmp[0];
    __syncthreads();  // every thread has read tmp[0] before a later scan reuses tmp
    return total;
  }
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int acc = kMax ? INT_MIN : 0;
  for (int i = lo; i < hi; ++i) acc = kMax ? max(acc, a[i]) : acc + a[i];
  tmp[tid] = acc;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 256 run totals
  for (int off = 1; off < kThreads; off <<= 1) {
    int v = tid >= off ? tmp[tid - off] : (kMax ? INT_MIN : 0);
    __syncthreads();
    if (tid >= off) tmp[tid] = kMax ? max(tmp[tid], v) : tmp[tid] + v;
    __syncthreads();
  }
  int carry = tid ? tmp[tid - 1] : (kMax ? INT_MIN : 0);
  const int total = tmp[kThreads - 1];
  for (int i = lo; i < hi; ++i) {
    if (kMax) {
      carry = max(carry, a[i]);
      a[i] = carry;
    } else {
      const int v = a[i];
      a[i] = carry;
      carry += v;
    }
  }
  __syncthreads();
  return total;
}

}  // namespace moe
