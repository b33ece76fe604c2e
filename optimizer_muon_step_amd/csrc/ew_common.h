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

}  // namespace ew
}  // namespace muon
