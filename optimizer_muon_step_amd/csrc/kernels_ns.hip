// POLY and UPDATE launches of the Newton-Schulz core (ns_gemm_tile.h), the
// reduce pass of cut Gram tiles, and the launch dispatch.  The Gram kernel is
// compiled in kernels_ns_gram.hip, a translation unit of its own, so that it
// can be built with its own instruction-scheduling options.
#include "ns_gemm_tile.h"

namespace muon {

hipError_t launch_gemm(int kind, const MatDesc* d, const GemmItem* items, int n_items, int src,
                       float ca, float cb, float cc, float* part, int tile, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  switch (kind) {
    case GEMM_GRAM:
      return launch_gemm_gram(d, items, n_items, src, part, tile, s);
    case GEMM_POLY:
      if (tile == TILE_MEDIUM)
        ns_gemm_kernel<GEMM_POLY, MED_POLY_BM, MED_POLY_BM, 2, 2, MED_POLY_NSTAGE, MED_POLY_BM, 64, false>
            <<<n_items, 256, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      else if (tile == TILE_SMALL)
        ns_gemm_kernel<GEMM_POLY, SMALL_SYM, SMALL_SYM, 2, 2, SMALL_SYM_NSTAGE, SMALL_SYM, 64, false>
            <<<n_items, 256, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      else
        ns_gemm_kernel<GEMM_POLY, SYM_BM, SYM_BN, 2, 4, SYM_NSTAGE, SYM_BM, SYM_BK, false>
            <<<n_items, 512, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      break;
    default:
      if (tile == TILE_MEDIUM)
        ns_gemm_kernel<GEMM_UPDATE, MED_UPD_BM, MED_UPD_BN, 2, 4, 2, UPD_ROWU, 64, false>
            <<<n_items, 512, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      else if (tile == TILE_SMALL)
        ns_gemm_kernel<GEMM_UPDATE, SMALL_UPD_BM, SMALL_UPD_BN, 2, 2, SMALL_UPD_NSTAGE, UPD_ROWU, 64, false>
            <<<n_items, 256, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      else if (tile == TILE_SHALLOW)
        ns_gemm_kernel<GEMM_UPDATE, SMALL_UPD_BM, SMALL_UPD_BN, 2, 2, SHALLOW_UPD_NSTAGE, UPD_ROWU, 64, false>
            <<<n_items, 256, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      else
        ns_gemm_kernel<GEMM_UPDATE, UPD_BM, UPD_BN, 2, 4, 2, UPD_ROWU, 64, true>
            <<<n_items < UPD_BLOCKS ? n_items : UPD_BLOCKS, 512, 0, s>>>(d, items, src, ca, cb, cc, n_items, part);
      break;
  }
  return hipGetLastError();
}

// Reduce pass of split Gram tiles (bm x bm, GRAM_BM or MED_GRAM_BM): one
// block per 64x64 sub-tile.  Each
// element sums its tile's chunk partials in K order in fp32, is rounded once
// to bf16, and is written at (r, c) and mirrored to (c, r); a diagonal tile
// keeps the values on and above its diagonal, so A stays exactly symmetric.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const MatDesc* __restrict__ descs,
                                                          const RedItem* __restrict__ items,
                                                          const float* __restrict__ part, int bm) {
  constexpr int T = RED_TILE;
  __shared__ uint16_t tile[T][T + 2];
  const RedItem it = items[blockIdx.x];
  const MatDesc& d = descs[it.mat];
  MUON_GLOBAL uint16_t* A = gptr(d.A);
  const int ld = d.ld_a;
  const int r0 = it.ti * bm + it.bi * T, c0 = it.tj * bm + it.bj * T;  // of A
  const int i = threadIdx.x >> 2, j0 = (threadIdx.x & 3) * 16;                    // within the sub-tile
  const float* src = part + (size_t)it.slot0 * (bm * bm) + (it.bi * T + i) * bm + it.bj * T + j0;
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = 0.0f;
  for (int c = 0; c < it.nchunk; ++c) {
    const float4* p = reinterpret_cast<const float4*>(src + (size_t)c * (bm * bm));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = p[q];
      v[4 * q] += t.x;
      v[4 * q + 1] += t.y;
      v[4 * q + 2] += t.z;
      v[4 * q + 3] += t.w;
    }
  }
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    tile[i][j0 + 2 * k] = (uint16_t)(w[k] & 0xffffu);
    tile[i][j0 + 2 * k + 1] = (uint16_t)(w[k] >> 16);
  }
  const int r = r0 + i;
  if (r <= c0 + j0) {
    // the whole run lies on or above the diagonal
    *reinterpret_cast<MUON_GLOBAL u32x4*>(A + (int64_t)r * ld + c0 + j0) =
        u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<MUON_GLOBAL u32x4*>(A + (int64_t)r * ld + c0 + j0 + 8) =
        u32x4{w[4], w[5], w[6], w[7]};
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (r <= c0 + j0 + k) A[(int64_t)r * ld + c0 + j0 + k] = tile[i][j0 + k];
  }
  __syncthreads();
  // mirror: row c0 + i of A takes column i of the sub-tile, strictly below
  // the diagonal
  const int mr = c0 + i;
  if (r0 + j0 + 15 < mr) {
    uint32_t m[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) m[k] = (uint32_t)tile[j0 + 2 * k][i] | ((uint32_t)tile[j0 + 2 * k + 1][i] << 16);
    *reinterpret_cast<MUON_GLOBAL u32x4*>(A + (int64_t)mr * ld + r0 + j0) = u32x4{m[0], m[1], m[2], m[3]};
    *reinterpret_cast<MUON_GLOBAL u32x4*>(A + (int64_t)mr * ld + r0 + j0 + 8) = u32x4{m[4], m[5], m[6], m[7]};
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int mc = r0 + j0 + k;
      if (mc < mr) A[(int64_t)mr * ld + mc] = tile[j0 + k][i];
    }
  }
}

hipError_t launch_gram_reduce(const MatDesc* d, const RedItem* items, int n_items, const float* part, int bm,
                              hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  gram_reduce_kernel<<<n_items, 256, 0, s>>>(d, items, part, bm);
  return hipGetLastError();
}

}  // namespace muon
