// HBM-bound kernels of the Muon step on gfx950:
//   momentum  M <- beta M + G ; U = G + beta M ; per-matrix sum of U^2 (fp64)
//   cast      X0 = bf16(U * s), s = 1 / (||U||_F + 1e-7), canonical (m <= n)
//             padded layout, transposed through LDS for tall matrices
//   apply     W <- W - lr * X (transposed back through LDS), optional bf16 copy
// Momentum convention: SGD with a running sum (the "Momentum" section of
// "07. Training neural networks" notes PyTorch's form without the (1 - beta)
// factor); the Nesterov look-ahead and the orthogonalisation order follow the
// "new optimizer" thread, tweet 5/8.  Every fp32 operation here is one IEEE
// rounding: the library is built with -ffp-contract=off so no product is fused
// into a sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_util.h"
#include "muon_internal.h"

namespace muon {

namespace {

constexpr int kWaves = EW_THREADS / 64;

// Fixed-order block sum of one double per thread; the total is valid in thread 0.
__device__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w];
  }
  return s;
}

__device__ __forceinline__ float nesterov(float g, float m_new, float beta) {
  return g + beta * m_new;
}

}  // namespace

// One work item = MOM_CHUNK consecutive elements of one matrix.  The block
// that finishes last for a matrix (counted with a device-scope atomic) sums
// that matrix's partials in index order and stores s, so the result does not
// depend on scheduling.
__global__ __launch_bounds__(EW_THREADS) void momentum_kernel(const MatDesc* __restrict__ descs,
                                                              const EwItem* __restrict__ items,
                                                              float beta) {
  __shared__ double red[kWaves];
  __shared__ int is_last;
  const EwItem it = items[blockIdx.x];
  const MatDesc& d = descs[it.mat];
  const int64_t total = (int64_t)d.rows * d.cols;
  const int64_t base = (int64_t)it.idx * MOM_CHUNK;
  const int64_t end = min(base + (int64_t)MOM_CHUNK, total);
  const float* __restrict__ G = d.G;
  float* __restrict__ M = d.M;
  double ss = 0.0;
  int64_t scalar_from = base;
  if (d.vec4) {
    const int n4 = (int)((end - base) >> 2);
    const float4* __restrict__ g4 = reinterpret_cast<const float4*>(G + base);
    float4* __restrict__ m4 = reinterpret_cast<float4*>(M + base);
#pragma unroll 4
    for (int k = threadIdx.x; k < n4; k += EW_THREADS) {
      const float4 g = g4[k];
      float4 m = m4[k];
      m.x = beta * m.x + g.x;
      m.y = beta * m.y + g.y;
      m.z = beta * m.z + g.z;
      m.w = beta * m.w + g.w;
      m4[k] = m;
      const float ux = nesterov(g.x, m.x, beta), uy = nesterov(g.y, m.y, beta);
      const float uz = nesterov(g.z, m.z, beta), uw = nesterov(g.w, m.w, beta);
      ss += (double)ux * ux;
      ss += (double)uy * uy;
      ss += (double)uz * uz;
      ss += (double)uw * uw;
    }
    scalar_from = base + ((int64_t)n4 << 2);
  }
  for (int64_t e = scalar_from + threadIdx.x; e < end; e += EW_THREADS) {
    const float g = G[e];
    const float m = beta * M[e] + g;
    M[e] = m;
    const float u = nesterov(g, m, beta);
    ss += (double)u * u;
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) {
    d.part[it.idx] = ss;
    __threadfence();
    const unsigned prev = atomicAdd(d.counter, 1u);
    is_last = (prev == (unsigned)(d.part_cnt - 1));
  }
  __syncthreads();
  if (is_last) {
    __threadfence();
    double v = 0.0;
    for (int k = threadIdx.x; k < d.part_cnt; k += EW_THREADS) v += __builtin_nontemporal_load(&d.part[k]);
    __syncthreads();
    v = block_sum(v, red);
    if (threadIdx.x == 0) {
      *d.scale = (float)(1.0 / (sqrt(v) + 1e-7));
      *d.counter = 0u;  // leave the counter at rest for the next call
    }
  }
}

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
      const uint2 w = *reinterpret_cast<const uint2*>(d.xin + off);
      out[0] = bf16_lo(w.x);
      out[1] = bf16_hi(w.x);
      out[2] = bf16_lo(w.y);
      out[3] = bf16_hi(w.y);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[k] = (c + k < d.cols) ? bf16_bits_to_f32(d.xin[off + k]) : 0.0f;
    }
    return;
  }
  float g[4], m[4];
  if (d.vec4 && c + 3 < d.cols) {
    const float4 g4 = *reinterpret_cast<const float4*>(d.G + off);
    const float4 m4 = *reinterpret_cast<const float4*>(d.M + off);
    g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
    m[0] = m4.x; m[1] = m4.y; m[2] = m4.z; m[3] = m4.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = c + k < d.cols;
      g[k] = in ? d.G[off + k] : 0.0f;
      m[k] = in ? d.M[off + k] : 0.0f;
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
  uint16_t* __restrict__ X = d.X[0];
  const int tc = (threadIdx.x & 15) * 4;
  const int tr = threadIdx.x >> 4;
  if (!d.transposed) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + tr + 16 * q;
      const int j = j0 + tc;
      float v[4];
      load4_src<FROM_BF16>(d, i, j, beta, s, v);
      uint2 w;
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(X + (int64_t)i * d.n_pad + j) = w;
    }
  } else {
    // canonical (i, j) comes from source (j, i): stage a source tile whose
    // rows are canonical columns j0.. and columns are canonical rows i0..
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
      load4_src<FROM_BF16>(d, j0 + tr + 16 * q, i0 + tc, beta, s, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) T[tr + 16 * q][tc + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = tr + 16 * q;
      uint2 w;
      w.x = pack_bf16x2(T[tc + 0][il], T[tc + 1][il]);
      w.y = pack_bf16x2(T[tc + 2][il], T[tc + 3][il]);
      *reinterpret_cast<uint2*>(X + (int64_t)(i0 + il) * d.n_pad + j0 + tc) = w;
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
  const uint16_t* __restrict__ X = d.X[src];
  const int tc = (threadIdx.x & 15) * 4;
  const int tr = threadIdx.x >> 4;
  uint32_t h[4][4];
  if (!d.transposed) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = min(r0 + tr + 16 * q, d.m_pad - 1);
      const uint2 w = *reinterpret_cast<const uint2*>(X + (int64_t)r * d.n_pad + c0 + tc);
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
      const uint2 w = *reinterpret_cast<const uint2*>(X + (int64_t)xr * d.n_pad + r0 + tc);
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
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + tr + 16 * q;
    const int c = c0 + tc;
    if (r >= d.rows) continue;
    const int64_t off = (int64_t)r * d.cols + c;
    if (write_w) {
      if (d.vec4 && c + 3 < d.cols) {
        float4 w = *reinterpret_cast<const float4*>(d.W + off);
        w.x = w.x - lr * bf16_bits_to_f32(h[q][0]);
        w.y = w.y - lr * bf16_bits_to_f32(h[q][1]);
        w.z = w.z - lr * bf16_bits_to_f32(h[q][2]);
        w.w = w.w - lr * bf16_bits_to_f32(h[q][3]);
        *reinterpret_cast<float4*>(d.W + off) = w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c + k < d.cols) d.W[off + k] = d.W[off + k] - lr * bf16_bits_to_f32(h[q][k]);
      }
    }
    if (d.upd) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (c + k < d.cols) d.upd[off + k] = (uint16_t)h[q][k];
    }
  }
}

hipError_t launch_momentum(const MatDesc* d, const EwItem* items, int n_items, float beta,
                           hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  momentum_kernel<<<n_items, EW_THREADS, 0, s>>>(d, items, beta);
  return hipGetLastError();
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
