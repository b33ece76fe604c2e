// Momentum pass of the Muon step on gfx950 (HBM-bound):
//   M <- beta M + G ; U = G + beta M ; per-matrix sum of U^2 (fp64)
// and the per-matrix finalisation of the Frobenius scale.  Momentum
// convention: SGD with a running sum (the "Momentum" section of "07. Training
// neural networks" notes PyTorch's form without the (1 - beta) factor); the
// Nesterov look-ahead follows the "new optimizer" thread, tweet 5/8.  Every
// fp32 operation here is one IEEE rounding: the library is built with
// -ffp-contract=off so no product is fused into a sum.  A translation unit of
// its own so that the build can schedule it apart from cast and apply.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16_util.h"
#include "ew_common.h"
#include "muon_internal.h"

namespace muon {

using namespace ew;

// One work item = MOM_CHUNK consecutive elements of one matrix (blocks take
// the items in per-XCD runs of EW_MOM_RUN, ew_item_of_block); it writes one
// fp64 partial sum of U^2, at the item's own slot.  The partials of a matrix are then reduced in one
// fixed order (norm_scale: by norm_finalize_kernel, or by each cast block for
// matrices of at most NORM_FOLD_MAX partials), so the result does not depend
// on scheduling (and no device-scope fence is needed inside the streaming
// kernel).  All loads of a
// batch are issued before any store so the whole batch is in flight at once.
// G and M are read with non-temporal loads (measured 15% faster than cached
// ones).  The new M is stored normally: the cast pass reads it again right
// after, and part of it is still in the memory-side cache then (cast 136
// against 149 us, momentum 170 against 168).
__global__ __launch_bounds__(EW_THREADS) void momentum_kernel(const MatDesc* __restrict__ descs,
                                                              const EwItem* __restrict__ items,
                                                              float beta) {
  constexpr int V = MOM_CHUNK / (4 * EW_THREADS);  // float4 per thread
  __shared__ double red[kWaves];
  const EwItem it = items[ew_item_of_block(blockIdx.x, gridDim.x, EW_MOM_RUN)];
  const MatDesc& d = descs[it.mat];
  const int64_t total = (int64_t)d.rows * d.cols;
  const int64_t base = (int64_t)it.idx * MOM_CHUNK;
  const int64_t end = min(base + (int64_t)MOM_CHUNK, total);
  const MUON_GLOBAL float* G = gptr(d.G);
  MUON_GLOBAL float* M = gptr(d.M);
  double ss = 0.0;
  if (d.vec4 && end - base == MOM_CHUNK) {
    const MUON_GLOBAL f32x4* g4 = reinterpret_cast<const MUON_GLOBAL f32x4*>(G + base);
    MUON_GLOBAL f32x4* m4 = reinterpret_cast<MUON_GLOBAL f32x4*>(M + base);
    f32x4 g[V], m[V];
#pragma unroll
    for (int v = 0; v < V; ++v) g[v] = __builtin_nontemporal_load(&g4[v * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int v = 0; v < V; ++v) m[v] = __builtin_nontemporal_load(&m4[v * EW_THREADS + threadIdx.x]);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      m[v].x = beta * m[v].x + g[v].x;
      m[v].y = beta * m[v].y + g[v].y;
      m[v].z = beta * m[v].z + g[v].z;
      m[v].w = beta * m[v].w + g[v].w;
      m4[v * EW_THREADS + threadIdx.x] = m[v];
      const float ux = nesterov(g[v].x, m[v].x, beta), uy = nesterov(g[v].y, m[v].y, beta);
      const float uz = nesterov(g[v].z, m[v].z, beta), uw = nesterov(g[v].w, m[v].w, beta);
      ss += (double)ux * ux;
      ss += (double)uy * uy;
      ss += (double)uz * uz;
      ss += (double)uw * uw;
    }
  } else {
    // partial or unaligned chunk: scalar elements, batches of 4V per thread
    for (int64_t b0 = base; b0 < end; b0 += 4 * V * EW_THREADS) {
      float g[4 * V], m[4 * V];
#pragma unroll
      for (int v = 0; v < 4 * V; ++v) {
        const int64_t e = b0 + v * EW_THREADS + threadIdx.x;
        g[v] = e < end ? G[e] : 0.0f;
        m[v] = e < end ? M[e] : 0.0f;
      }
#pragma unroll
      for (int v = 0; v < 4 * V; ++v) {
        const int64_t e = b0 + v * EW_THREADS + threadIdx.x;
        if (e < end) {
          const float mn = beta * m[v] + g[v];
          M[e] = mn;
          const float u = nesterov(g[v], mn, beta);
          ss += (double)u * u;
        }
      }
    }
  }
  ss = block_sum(ss, red);
  if (threadIdx.x == 0) d.part[it.idx] = ss;
}

// One block per matrix of the list (those with more than NORM_FOLD_MAX
// partials): its scale s = 1 / (sqrt(sum of partials) + 1e-7).
__global__ __launch_bounds__(EW_THREADS) void norm_finalize_kernel(const MatDesc* __restrict__ descs,
                                                                   const int32_t* __restrict__ fin) {
  __shared__ double red[kWaves];
  const MatDesc& d = descs[fin[blockIdx.x]];
  const float s = norm_scale(d, red);
  if (threadIdx.x == 0) *d.scale = s;
}

hipError_t launch_momentum(const MatDesc* d, const EwItem* items, int n_items, const int32_t* fin, int n_fin,
                           float beta, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  momentum_kernel<<<n_items, EW_THREADS, 0, s>>>(d, items, beta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_fin == 0) return e;
  norm_finalize_kernel<<<n_fin, EW_THREADS, 0, s>>>(d, fin);
  return hipGetLastError();
}

}  // namespace muon
