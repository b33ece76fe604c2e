// Multi-tensor AdamW step on gfx950 (HBM-bound, elementwise).
//
// For every element of every tensor of a call (the "07. Training neural
// networks" page, section "Adam, weight decay and AdamW", with the decoupled
// decay of its derivation block):
//   p1 = p * (1 - lr*lambda)                      decay first, per tensor lambda
//   u' = beta1*u + (1-beta1)*g
//   v' = beta2*v + ((1-beta2)*g)*g
//   p' = p1 - (lr * (u'/bc1)) / (sqrt(v'/bc2) + eps),  bc_i = 1 - beta_i^t
// Every operation is one IEEE fp32 rounding in that order: the library is
// built with -ffp-contract=off (no fused multiply-add) and HIP's default
// correctly rounded fp32 division and square root.  The per-call constants
// (1-beta_i, bc_i) arrive precomputed from the host.
//
// Work list: one item per ADAM_CHUNK consecutive elements of one tensor, so a
// launch covers tensors of any mix of sizes.  p, g, u and v are each read
// once and p, u, v written once (28 bytes per element); the streams have no
// reuse, so they are loaded and stored non-temporally.  A full chunk of a
// tensor whose four arrays are 16-byte aligned moves as float4, all loads of
// the chunk issued before any arithmetic; other chunks go element by element.
//
// Also here: the transposed copy of a parameter and its moments used when a
// tied embedding / output layer pair is untied.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_util.h"
#include "muon_internal.h"

namespace muon {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void adamw_elem(float& p, float g, float& u, float& v, const AdamConst& c,
                                           float decay) {
  const float p1 = p * decay;
  const float u1 = c.beta1 * u + c.omb1 * g;
  const float v1 = c.beta2 * v + (c.omb2 * g) * g;
  const float uh = u1 / c.bc1;
  const float vh = v1 / c.bc2;
  const float den = sqrtf(vh) + c.eps;
  p = p1 - (c.lr * uh) / den;
  u = u1;
  v = v1;
}

}  // namespace

__global__ __launch_bounds__(EW_THREADS) void adamw_kernel(const AdamDesc* __restrict__ descs,
                                                           const EwItem* __restrict__ items, AdamConst c) {
  constexpr int V = ADAM_CHUNK / (4 * EW_THREADS);  // float4 per thread per array
  const EwItem it = items[blockIdx.x];
  const AdamDesc& d = descs[it.mat];
  const int64_t base = (int64_t)it.idx * ADAM_CHUNK;
  const int64_t end = min(base + (int64_t)ADAM_CHUNK, d.numel);
  const float decay = 1.0f - c.lr * (d.wd_shared ? c.wd_shared : d.wd);
  MUON_GLOBAL float* P = gptr(d.p);
  const MUON_GLOBAL float* G = gptr(d.g);
  MUON_GLOBAL float* U = gptr(d.u);
  MUON_GLOBAL float* Q = gptr(d.v);
  if (d.vec4 && end - base == ADAM_CHUNK) {
    MUON_GLOBAL f32x4* p4 = reinterpret_cast<MUON_GLOBAL f32x4*>(P + base);
    const MUON_GLOBAL f32x4* g4 = reinterpret_cast<const MUON_GLOBAL f32x4*>(G + base);
    MUON_GLOBAL f32x4* u4 = reinterpret_cast<MUON_GLOBAL f32x4*>(U + base);
    MUON_GLOBAL f32x4* v4 = reinterpret_cast<MUON_GLOBAL f32x4*>(Q + base);
    f32x4 p[V], g[V], u[V], v[V];
#pragma unroll
    for (int k = 0; k < V; ++k) g[k] = __builtin_nontemporal_load(&g4[k * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int k = 0; k < V; ++k) u[k] = __builtin_nontemporal_load(&u4[k * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = __builtin_nontemporal_load(&v4[k * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int k = 0; k < V; ++k) p[k] = __builtin_nontemporal_load(&p4[k * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int k = 0; k < V; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[k][e], ue = u[k][e], ve = v[k][e];
        adamw_elem(pe, g[k][e], ue, ve, c, decay);
        p[k][e] = pe;
        u[k][e] = ue;
        v[k][e] = ve;
      }
      __builtin_nontemporal_store(u[k], &u4[k * EW_THREADS + threadIdx.x]);
      __builtin_nontemporal_store(v[k], &v4[k * EW_THREADS + threadIdx.x]);
      __builtin_nontemporal_store(p[k], &p4[k * EW_THREADS + threadIdx.x]);
    }
  } else {
    // tail or unaligned chunk: one element per thread per pass
    for (int64_t e = base + threadIdx.x; e < end; e += EW_THREADS) {
      float pe = P[e], ue = U[e], ve = Q[e];
      adamw_elem(pe, G[e], ue, ve, c, decay);
      P[e] = pe;
      U[e] = ue;
      Q[e] = ve;
    }
  }
}

// Delayed untying: copy a shared parameter and its two AdamW moments into
// new buffers, transposed (rows x cols -> cols x rows).  One 64x64 tile per
// block and array; rows are read and written as whole 256-byte segments, the
// transpose happens in LDS (row stride 65 words, so the column reads of the
// write-out hit 64 different banks).
constexpr int UNTIE_TILE = 64;

__global__ __launch_bounds__(EW_THREADS) void untie_transpose_kernel(UntieArgs a, int64_t rows, int64_t cols,
                                                                     int64_t tiles_c) {
  __shared__ float tile[UNTIE_TILE][UNTIE_TILE + 1];
  const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int64_t r0 = tr * UNTIE_TILE, c0 = tc * UNTIE_TILE;
  const int lx = threadIdx.x % UNTIE_TILE, ly = threadIdx.x / UNTIE_TILE;  // 64 x 4 threads
  for (int k = 0; k < 3; ++k) {
    const MUON_GLOBAL float* src = gptr(a.src[k]);
    MUON_GLOBAL float* dst = gptr(a.dst[k]);
    for (int y = ly; y < UNTIE_TILE; y += EW_THREADS / UNTIE_TILE) {
      const int64_t r = r0 + y, c = c0 + lx;
      if (r < rows && c < cols) tile[y][lx] = src[r * cols + c];
    }
    __syncthreads();
    for (int y = ly; y < UNTIE_TILE; y += EW_THREADS / UNTIE_TILE) {
      const int64_t r = c0 + y, c = r0 + lx;  // destination row = source column
      if (r < cols && c < rows) dst[r * rows + c] = tile[lx][y];
    }
    __syncthreads();
  }
}

hipError_t launch_untie_transpose(const UntieArgs& a, int64_t rows, int64_t cols, hipStream_t s) {
  const int64_t tiles_r = (rows + UNTIE_TILE - 1) / UNTIE_TILE, tiles_c = (cols + UNTIE_TILE - 1) / UNTIE_TILE;
  if (tiles_r * tiles_c == 0) return hipSuccess;
  untie_transpose_kernel<<<(unsigned)(tiles_r * tiles_c), EW_THREADS, 0, s>>>(a, rows, cols, tiles_c);
  return hipGetLastError();
}

hipError_t launch_adamw(const AdamDesc* d, const EwItem* items, int n_items, const AdamConst& c, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  adamw_kernel<<<n_items, EW_THREADS, 0, s>>>(d, items, c);
  return hipGetLastError();
}

}  // namespace muon
