// bfloat16 helpers for gfx950 device code.
//
// bfloat16 is the upper half of an IEEE binary32 word.  Conversion rounds to
// nearest, ties to even, on the bit pattern; NaNs stay NaN (quiet bit set),
// infinities and overflow follow IEEE rounding.  Written out rather than left
// to the compiler so the rounding is fixed regardless of the FP mode register.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Pointers read out of descriptors are generic (flat) pointers; flat memory
// instructions also count against the LDS wait counter, so a pending global
// prefetch would stall every LDS wait.  Casting to the global address space
// makes the compiler emit global_load / global_store.
#define MUON_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ MUON_GLOBAL T* gptr(T* p) {
  return (MUON_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ const MUON_GLOBAL T* gptr(const T* p) {
  return (const MUON_GLOBAL T*)p;
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x40u;
  // select, not branch: this runs once per element of every epilogue
  return ((u & 0x7fffffffu) > 0x7f800000u) ? quiet_nan : rounded;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Two floats -> one dword holding two bf16 (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace muon
