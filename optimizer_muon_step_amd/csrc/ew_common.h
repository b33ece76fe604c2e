// Shared pieces of the elementwise kernels (momentum, cast, apply).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {
namespace ew {

constexpr int kWaves = EW_THREADS / 64;

// Native vector types: HIP's float4/uint2 classes cannot be assigned through
// global-address-space pointers.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The Nesterov look-ahead U = G + beta M on the updated buffer; the momentum
// pass (for the norm) and the cast pass (for X0) both take U from here.
__device__ __forceinline__ float nesterov(float g, float m_new, float beta) {
  return g + beta * m_new;
}

// Block barrier that waits for this wave's LDS operations only, so global
// loads in flight stay in flight across it (__syncthreads would wait for
// them too).  s_waitcnt immediate (gfx9 encoding): vmcnt 63 (no wait),
// expcnt 7 (no wait), lgkmcnt 0.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Fixed-order block sum of one double per thread; the total is valid in
// thread 0.  Every thread of the block calls it.  KEEP_LOADS: synchronise
// with lds_barrier (global loads issued before stay in flight); the sum is
// the same either way.
template <bool KEEP_LOADS = false>
__device__ __forceinline__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  if (KEEP_LOADS) lds_barrier(); else __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w];
  }
  return s;
}

// s = 1 / (sqrt(sum of the matrix's norm partials) + 1e-7), valid in thread
// 0.  The partials are summed in one fixed order (thread t takes partials t,
// t + EW_THREADS, ..., then the block sum), whichever kernel calls it.
template <bool KEEP_LOADS = false>
__device__ __forceinline__ float norm_scale(const MatDesc& d, double* red) {
  double v = 0.0;
  for (int k = threadIdx.x; k < d.part_cnt; k += EW_THREADS) v += d.part[k];
  v = block_sum<KEEP_LOADS>(v, red);
  return (float)(1.0 / (sqrt(v) + 1e-7));
}

}  // namespace ew
}  // namespace muon
