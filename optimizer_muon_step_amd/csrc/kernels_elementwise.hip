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

// Four bf16 input elements (r, c .. c+3) of the Newton-Schulz-only entry as
// fp32, zero outside the matrix.
__device__ __forceinline__ void load4_xin(const MatDesc& d, int r, int c, float out[4]) {
  if (r >= d.rows) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = 0.0f;
    return;
  }
  const int64_t off = (int64_t)r * d.cols + c;
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
}

// Four fp32 elements (r, c .. c+3) of G or M, zero outside the matrix; read
// non-temporally (their last use in the step).
__device__ __forceinline__ f32x4 load4_edge(const MUON_GLOBAL float* a, const MatDesc& d, int r, int c) {
  f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (r >= d.rows) return v;
  const int64_t off = (int64_t)r * d.cols + c;
  if (d.vec4 && c + 3 < d.cols) return __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(a + off));
  v.x = c < d.cols ? a[off] : 0.0f;
  v.y = c + 1 < d.cols ? a[off + 1] : 0.0f;
  v.z = c + 2 < d.cols ? a[off + 2] : 0.0f;
  v.w = c + 3 < d.cols ? a[off + 3] : 0.0f;
  return v;
}

// One work item = one tile of the canonical padded X0 (blocks take the items
// in per-XCD runs of EW_TILE_RUN, ew_item_of_block): CAST_WIDE_ROWS x
// CAST_WIDE_COLS for an untransposed matrix, CAST_TILE x CAST_TILE staged
// through LDS for a transposed one.  G and M go out first, eight 16-byte
// loads per thread in one batch on interior tiles, and the norm scale is
// taken while they are in flight.
template <bool FROM_BF16>
__global__ __launch_bounds__(EW_THREADS) void cast_kernel(const MatDesc* __restrict__ descs,
                                                          const EwItem* __restrict__ items,
                                                          float beta) {
  __shared__ float T[CAST_TILE][CAST_TILE + 1];
  const EwItem it = items[ew_item_of_block(blockIdx.x, gridDim.x, EW_TILE_RUN)];
  const MatDesc& d = descs[it.mat];
  const bool trn = d.transposed;
  // tile origin (i0, j0) in X0; this thread's source rows sr0 + tr + rstep q
  // (q = 0..3), columns sc0 + tc .. +3
  int i0, j0, tr, tc, rstep, srows, scols;
  if (!trn) {
    const int tiles_j = d.n_pad / CAST_WIDE_COLS;
    i0 = (it.idx / tiles_j) * CAST_WIDE_ROWS;
    j0 = (it.idx % tiles_j) * CAST_WIDE_COLS;
    tc = (threadIdx.x % (CAST_WIDE_COLS / 4)) * 4;
    tr = threadIdx.x / (CAST_WIDE_COLS / 4);
    rstep = CAST_WIDE_ROWS / 4;
    srows = CAST_WIDE_ROWS;
    scols = CAST_WIDE_COLS;
  } else {
    const int tiles_j = d.n_pad / CAST_TILE;
    i0 = (it.idx / tiles_j) * CAST_TILE;
    j0 = (it.idx % tiles_j) * CAST_TILE;
    tc = (threadIdx.x % (CAST_TILE / 4)) * 4;
    tr = threadIdx.x / (CAST_TILE / 4);
    rstep = CAST_TILE / 4;
    srows = scols = CAST_TILE;
  }
  const int sr0 = trn ? j0 : i0, sc0 = trn ? i0 : j0;
  float v[4][4];
  if (!FROM_BF16) {
    f32x4 g4[4], m4[4];
    if (d.vec4 && sr0 + srows <= d.rows && sc0 + scols <= d.cols) {
      const MUON_GLOBAL float* G = gptr(d.G) + (int64_t)(sr0 + tr) * d.cols + sc0 + tc;
      const MUON_GLOBAL float* Mp = gptr(d.M) + (int64_t)(sr0 + tr) * d.cols + sc0 + tc;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        g4[q] = __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(G + (int64_t)rstep * q * d.cols));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m4[q] = __builtin_nontemporal_load(reinterpret_cast<const MUON_GLOBAL f32x4*>(Mp + (int64_t)rstep * q * d.cols));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        g4[q] = load4_edge(gptr(d.G), d, sr0 + tr + rstep * q, sc0 + tc);
        m4[q] = load4_edge(gptr(d.M), d, sr0 + tr + rstep * q, sc0 + tc);
      }
    }
    // the norm scale: summed here from the matrix's partials when it has few
    // (the finalisation kernel's order, so the same bits), else its result
    float s;
    if (d.part_cnt <= NORM_FOLD_MAX) {
      __shared__ double red[kWaves];
      __shared__ float s_fold;
      const float f = norm_scale<true>(d, red);
      if (threadIdx.x == 0) s_fold = f;
      lds_barrier();
      s = s_fold;
    } else {
      s = *d.scale;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool row_in = sr0 + tr + rstep * q < d.rows;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[q][k] = (row_in && sc0 + tc + k < d.cols) ? nesterov(g4[q][k], m4[q][k], beta) * s : 0.0f;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) load4_xin(d, sr0 + tr + rstep * q, sc0 + tc, v[q]);
  }
  MUON_GLOBAL uint16_t* X = gptr(d.X[0]);
  if (!trn) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2 w;
      w.x = pack_bf16x2(v[q][0], v[q][1]);
      w.y = pack_bf16x2(v[q][2], v[q][3]);
      *reinterpret_cast<MUON_GLOBAL u32x2*>(X + (int64_t)(i0 + tr + rstep * q) * d.ld_x + j0 + tc) = w;
    }
  } else {
    // canonical (i, j) comes from source (j, i): stage a source tile whose
    // rows are canonical columns j0.. and columns are canonical rows i0..
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) T[tr + rstep * q][tc + k] = v[q][k];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = tr + rstep * q;
      u32x2 w;
      w.x = pack_bf16x2(T[tc + 0][il], T[tc + 1][il]);
      w.y = pack_bf16x2(T[tc + 2][il], T[tc + 3][il]);
      *reinterpret_cast<MUON_GLOBAL u32x2*>(X + (int64_t)(i0 + il) * d.ld_x + j0 + tc) = w;
    }
  }
}

// One work item = one tile of the caller's W (items in per-XCD runs of
// EW_TILE_RUN, as in the cast): CAST_WIDE_ROWS x CAST_WIDE_COLS for an
// untransposed matrix, CAST_TILE x CAST_TILE (X staged through LDS) for a
// transposed one.
__global__ __launch_bounds__(EW_THREADS) void apply_kernel(const MatDesc* __restrict__ descs,
                                                           const EwItem* __restrict__ items, float lr,
                                                           int src, int write_w) {
  __shared__ uint16_t T[CAST_TILE][CAST_TILE + 2];
  const EwItem it = items[ew_item_of_block(blockIdx.x, gridDim.x, EW_TILE_RUN)];
  const MatDesc& d = descs[it.mat];
  int r0, c0, tr, tc, rstep;
  if (!d.transposed) {
    const int tiles_c = (d.cols + CAST_WIDE_COLS - 1) / CAST_WIDE_COLS;
    r0 = (it.idx / tiles_c) * CAST_WIDE_ROWS;
    c0 = (it.idx % tiles_c) * CAST_WIDE_COLS;
    tc = (threadIdx.x % (CAST_WIDE_COLS / 4)) * 4;
    tr = threadIdx.x / (CAST_WIDE_COLS / 4);
    rstep = CAST_WIDE_ROWS / 4;
  } else {
    const int tiles_c = (d.cols + CAST_TILE - 1) / CAST_TILE;
    r0 = (it.idx / tiles_c) * CAST_TILE;
    c0 = (it.idx % tiles_c) * CAST_TILE;
    tc = (threadIdx.x % (CAST_TILE / 4)) * 4;
    tr = threadIdx.x / (CAST_TILE / 4);
    rstep = CAST_TILE / 4;
  }
  const MUON_GLOBAL uint16_t* X = gptr(d.X[src]);
  uint32_t h[4][4];
  if (!d.transposed) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = min(r0 + tr + rstep * q, d.m_pad - 1);
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
      const int r = r0 + tr + rstep * q;
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
      const int r = r0 + tr + rstep * q;
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
      const int r = r0 + tr + rstep * q;
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
