// bfloat16 helpers for gfx950 device code.
//
// bfloat16 is the upper half of an IEEE binary32 word.  Conversion rounds to
// nearest, ties to even; NaNs stay NaN (quiet bit set), infinities and
// overflow follow IEEE rounding.
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

// gfx950's v_cvt_pk_bf16_f32 rounds two floats to bfloat16, nearest-even,
// and keeps NaNs NaN with the quiet bit set: on every one of the 2^32 input
// patterns it gives the same bits as adding 0x7fff plus the lowest kept bit
// and truncating (for a NaN: its upper half with bit 6 set).  The kernels run
// in the default FP mode (round to nearest even, denormals kept).
typedef float muon_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 muon_bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> one dword holding two bf16 (first in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(muon_f32x2{lo, hi}, muon_bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace muon
