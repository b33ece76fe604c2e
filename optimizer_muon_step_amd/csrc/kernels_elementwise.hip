// Cast and apply passes of the Muon step on gfx950 (HBM-bound):
//   cast      X0 = bf16(U * s), U = G + beta M (Nesterov look-ahead on the
//             updated buffer), s = 1 / (||U||_F + 1e-7), canonical (m <= n)
//             padded layout, transposed through LDS for tall matrices
//   apply     W <- W - lr * X (transposed back through LDS), optional bf16 copy
// The momentum pass, which produces M and the norm, is in kernels_momentum.hip.
// The orthogonalisation order follows the "new optimizer" thread, tweet 5/8.
// Every fp32 operation here is one IEEE rounding: the library is built with
// -ffp-contract=off so no product is fused into a sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_util.h"
#include "ew_common.h"
#include "muon_internal.h"

namespace muon {

using namespace ew;

// Value of canonical element (i, j) taken from source element (r, c); zero
// outside the matrix.
template <bool FROM_BF16>
__device__ __forceinline__ void load4_src(const MatDesc& d, int r, int c, float beta, float s,
                                          float out[4]) {
  if (r >= d.rows) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = 0.0f;
    return;
  }
  const int64_t off = (int64_t)r * d.cols + c;
  if (FROM_BF16) {
    if (d.vec4 && c + 3 < d.cols) {
      const u32x2 w = *reinterpret_cast<const MUON_GLOBAL u32x2*>(gptr(d.xin) + off);
      out[0] = bf16_lo(w.x);
      out[1] = bf16_hi(w.x);
      out[2] = bf16_lo(w.y);
      out[3] = bf16_hi(w.y);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = (c + k < d.cols) ? bf16_bits_to_f32(gptr(d.xin)[off + k]) : 0.0f;
    }
    return;
  }
  // G and M are read here for the last time in the step: non-temporal loads
  float g[4], m[4];
  if (d.vec4 && c + 3 < d.cols) {
    const f32x4 g4 = __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(gptr(d.G) + off));
    const f32x4 m4 = __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(gptr(d.M) + off));
    g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
    m[0] = m4.x; m[1] = m4.y; m[2] = m4.z; m[3] = m4.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = c + k < d.cols;
      g[k] = in ? gptr(d.G)[off + k] : 0.0f;
      m[k] = in ? gptr(d.M)[off + k] : 0.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = (c + k < d.cols) ? nesterov(g[k], m[k], beta) * s : 0.0f;
}

// One work item = one CAST_TILE x CAST_TILE tile of the canonical padded X0.
template <bool FROM_BF16>
__global__ __launch_bounds__(EW_THREADS) void cast_kernel(const MatDesc* __restrict__ descs,
                                                          const EwItem* __restrict__ items,
                                                          float beta) {
  __shared__ float T[CAST_TILE][CAST_TILE + 1];
  const EwItem it = items[blockIdx.x];
  const MatDesc& d = descs[it.mat];
  const int tiles_j = d.n_pad / CAST_TILE;
  const int i0 = (it.idx / tiles_j) * CAST_TILE;
  const int j0 = (it.idx % tiles_j) * CAST_TILE;
  const float s = FROM_BF16 ? 1.0f : *d.scale;
  MUON_GLOBAL uint16_t* X = gptr(d.X[0]);
  const int tc = (threadIdx.x & 15) * 4;
  const int tr = threadIdx.x >> 4;
  float v[4][4];
  if (!d.transposed) {
    // all loads first, then all stores
#pragma unroll
    for (int q = 0; q < 4; ++q) load4_src<FROM_BF16>(d, i0 + tr + 16 * q, j0 + tc, beta, s, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2 w;
      w.x = pack_bf16x2(v[q][0], v[q][1]);
      w.y = pack_bf16x2(v[q][2], v[q][3]);
      *reinterpret_cast<MUON_GLOBAL u32x2*>(X + (int64_t)(i0 + tr + 16 * q) * d.ld_x + j0 + tc) = w;
    }
  } else {
    // canonical (i, j) comes from source (j, i): stage a source tile whose
    // rows are canonical columns j0.. and columns are canonical rows i0..
#pragma unroll
    for (int q = 0; q < 4; ++q) load4_src<FROM_BF16>(d, j0 + tr + 16 * q, i0 + tc, beta, s, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) T[tr + 16 * q][tc + k] = v[q][k];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = tr + 16 * q;
      u32x2 w;
      w.x = pack_bf16x2(T[tc + 0][il], T[tc + 1][il]);
      w.y = pack_bf16x2(T[tc + 2][il], T[tc + 3][il]);
      *reinterpret_cast<MUON_GLOBAL u32x2*>(X + (int64_t)(i0 + il) * d.ld_x + j0 + tc) = w;
    }
  }
}

// One work item = one CAST_TILE x CAST_TILE tile of the caller's W.
__global__ __launch_bounds__(EW_THREADS) void apply_kernel(const MatDesc* __restrict__ descs,
                                                           const EwItem* __restrict__ items, float lr,
                                                           int src, int write_w) {
  __shared__ uint16_t T[CAST_TILE][CAST_TILE + 2];
  const EwItem it = items[blockIdx.x];
  const MatDesc& d = descs[it.mat];
  const int tiles_c = (d.cols + CAST_TILE - 1) / CAST_TILE;
  const int r0 = (it.idx / tiles_c) * CAST_TILE;
  const int c0 = (it.idx % tiles_c) * CAST_TILE;
  const MUON_GLOBAL uint16_t* X = gptr(d.X[src]);
  const int tc = (threadIdx.x & 15) * 4;
  const int tr = threadIdx.x >> 4;
  uint32_t h[4][4];
  if (!d.transposed) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = min(r0 + tr + 16 * q, d.m_pad - 1);
      const u32x2 w = *reinterpret_cast<const MUON_GLOBAL u32x2*>(X + (int64_t)r * d.ld_x + c0 + tc);
      h[q][0] = w.x & 0xffffu;
      h[q][1] = w.x >> 16;
      h[q][2] = w.y & 0xffffu;
      h[q][3] = w.y >> 16;
    }
  } else {
    // W(r, c) = X(c, r): stage the X tile with rows c0.. and columns r0..
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int xr = c0 + tr + 16 * q;
      const u32x2 w = *reinterpret_cast<const MUON_GLOBAL u32x2*>(X + (int64_t)xr * d.ld_x + r0 + tc);
      T[tr + 16 * q][tc + 0] = (uint16_t)(w.x & 0xffffu);
      T[tr + 16 * q][tc + 1] = (uint16_t)(w.x >> 16);
      T[tr + 16 * q][tc + 2] = (uint16_t)(w.y & 0xffffu);
      T[tr + 16 * q][tc + 3] = (uint16_t)(w.y >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) h[q][k] = T[tc + k][tr + 16 * q];
  }
  if (write_w) {
    MUON_GLOBAL float* W = gptr(d.W);
    const bool vec = d.vec4 && (c0 + tc + 3 < d.cols);
    // W is read and written once per step: non-temporal accesses
    float w[4][4];
    // all loads of W first, then the stores
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + tr + 16 * q;
      const int64_t off = (int64_t)r * d.cols + c0 + tc;
      if (r >= d.rows) continue;
      if (vec) {
        const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(W + off));
        w[q][0] = t.x; w[q][1] = t.y; w[q][2] = t.z; w[q][3] = t.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[q][k] = (c0 + tc + k < d.cols) ? W[off + k] : 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + tr + 16 * q;
      const int64_t off = (int64_t)r * d.cols + c0 + tc;
      if (r >= d.rows) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[q][k] = w[q][k] - lr * bf16_bits_to_f32(h[q][k]);
      if (vec) {
        __builtin_nontemporal_store(f32x4{w[q][0], w[q][1], w[q][2], w[q][3]}, reinterpret_cast<MUON_GLOBAL f32x4*>(W + off));
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c0 + tc + k < d.cols) W[off + k] = w[q][k];
      }
    }
  }
  if (d.upd) {
    MUON_GLOBAL uint16_t* U = gptr(d.upd);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = r0 + tr + 16 * q;
      const int c = c0 + tc;
      if (r >= d.rows) continue;
      const int64_t off = (int64_t)r * d.cols + c;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < d.cols) U[off + k] = (uint16_t)h[q][k];
    }
  }
}

hipError_t launch_cast(const MatDesc* d, const EwItem* items, int n_items, float beta, int from_bf16,
                       hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  if (from_bf16)
    cast_kernel<true><<<n_items, EW_THREADS, 0, s>>>(d, items, beta);
  else
    cast_kernel<false><<<n_items, EW_THREADS, 0, s>>>(d, items, beta);
  return hipGetLastError();
}

hipError_t launch_apply(const MatDesc* d, const EwItem* items, int n_items, float lr, int src,
                        int write_w, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  apply_kernel<<<n_items, EW_THREADS, 0, s>>>(d, items, lr, src, write_w);
  return hipGetLastError();
}

}  // namespace muon
