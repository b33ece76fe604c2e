// Internal declarations shared by the host plan code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_types.h"

namespace muon {

// ---- host launchers (kernels_*.hip) ----
hipError_t launch_momentum(const MatDesc* d, const EwItem* items, int n_items, const int32_t* fin, int n_fin,
                           float beta, hipStream_t s);
hipError_t launch_cast(const MatDesc* d, const EwItem* items, int n_items, float beta, int from_bf16,
                       hipStream_t s);
hipError_t launch_apply(const MatDesc* d, const EwItem* items, int n_items, float lr, int src,
                        int write_w, hipStream_t s);
// tile: the TileKind of the launch (large, small or medium tiles).
hipError_t launch_gemm(int kind, const MatDesc* d, const GemmItem* items, int n_items, int src,
                       float ca, float cb, float cc, float* part, int tile, hipStream_t s);
hipError_t launch_gemm_gram(const MatDesc* d, const GemmItem* items, int n_items, int src, float* part,
                            int tile, hipStream_t s);
// POLY and UPDATE of one iteration in one launch over the small update
// tiles, for calls whose matrices all have m_pad = FUSED_M_PAD.
hipError_t launch_poly_update(const MatDesc* d, const GemmItem* items, int n_items, int src, float ca, float cb,
                              float cc, hipStream_t s);
// bm: edge of the cut Gram tiles (and of their fp32 partial tiles).
hipError_t launch_gram_reduce(const MatDesc* d, const RedItem* items, int n_items, const float* part, int bm,
                              hipStream_t s);
// Table maintenance: write pointer records into descriptors, or a chunk of a
// table image to device memory, in stream order (kernels_tables.hip).
hipError_t launch_ptr_patch(MatDesc* descs, const PtrPatch& p, hipStream_t s);
hipError_t launch_blob_write(void* dst, const BlobChunk& c, hipStream_t s);
hipError_t launch_adamw(const AdamDesc* d, const EwItem* items, int n_items, const AdamConst& c, hipStream_t s);

// Source and destination of the three arrays (param, exp_avg, exp_avg_sq)
// of a delayed-untying copy.
struct UntieArgs {
  const float* src[3];
  float* dst[3];
};
hipError_t launch_untie_transpose(const UntieArgs& a, int64_t rows, int64_t cols, hipStream_t s);

}  // namespace muon
