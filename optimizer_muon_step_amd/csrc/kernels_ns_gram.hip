// GRAM launch of the Newton-Schulz core (ns_gemm_tile.h): A = bf16(X X^T),
// upper-triangle tiles mirrored on store.  A translation unit of its own so
// that the build can give this kernel its own instruction-scheduling options.
#include "ns_gemm_tile.h"

namespace muon {

hipError_t launch_gemm_gram(const MatDesc* d, const GemmItem* items, int n_items, int src, float* part,
                            int tile, hipStream_t s) {
  if (n_items == 0) return hipSuccess;
  if (tile == TILE_SMALL)
    ns_gemm_kernel<GEMM_GRAM, SMALL_SYM, SMALL_SYM, 2, 2, SMALL_SYM_NSTAGE, SMALL_SYM, 64, false>
        <<<n_items, 256, 0, s>>>(d, items, src, 0.0f, 0.0f, 0.0f, n_items, part);
  else if (tile == TILE_MEDIUM)
    ns_gemm_kernel<GEMM_GRAM, MED_GRAM_BM, MED_GRAM_BM, 2, 4, 2, MED_GRAM_BM, 64, false>
        <<<n_items, 512, 0, s>>>(d, items, src, 0.0f, 0.0f, 0.0f, n_items, part);
  else
    ns_gemm_kernel<GEMM_GRAM, GRAM_BM, GRAM_BM, 2, 4, 2, GRAM_BM, 64, false>
        <<<n_items, 512, 0, s>>>(d, items, src, 0.0f, 0.0f, 0.0f, n_items, part);
  return hipGetLastError();
}

}  // namespace muon
