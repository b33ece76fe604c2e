// Stream-ordered table maintenance for the host plan code.  Their payloads
// travel as kernel arguments (copied by value at launch, and held by a
// captured graph), so no host staging buffer, copy engine or synchronisation
// is involved.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

// Record t of the patch goes into descriptor rec[t].mat: the caller's
// pointers for this call and their vector-access flag.
__global__ __launch_bounds__(64) void ptr_patch_kernel(MatDesc* __restrict__ descs, const PtrPatch p) {
  const int t = threadIdx.x;
  if (t >= p.count) return;
  const PtrRecord r = p.rec[t];
  MatDesc* d = descs + r.mat;
  d->W = r.W;
  d->G = r.G;
  d->M = r.M;
  d->upd = r.upd;
  d->xin = r.xin;
  d->vec4 = r.vec4;
}

// c.words 32-bit words to dst (4-byte aligned).
__global__ __launch_bounds__(256) void blob_write_kernel(uint32_t* __restrict__ dst, const BlobChunk c) {
  for (int k = threadIdx.x; k < c.words; k += blockDim.x) dst[k] = c.w[k];
}

hipError_t launch_ptr_patch(MatDesc* descs, const PtrPatch& p, hipStream_t s) {
  if (p.count <= 0) return hipSuccess;
  ptr_patch_kernel<<<1, 64, 0, s>>>(descs, p);
  return hipGetLastError();
}

hipError_t launch_blob_write(void* dst, const BlobChunk& c, hipStream_t s) {
  if (c.words <= 0) return hipSuccess;
  blob_write_kernel<<<1, 256, 0, s>>>(static_cast<uint32_t*>(dst), c);
  return hipGetLastError();
}

}  // namespace muon
