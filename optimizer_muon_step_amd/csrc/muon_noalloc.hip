// muon_step_noalloc: the Muon step for callers that cannot allocate device
// memory.  Its workspace and plan tables live in one file-scope device
// array, `scratch`, of MUON_NOALLOC_SCRATCH_BYTES per device; the tables
// and the caller pointers reach the device as kernel arguments (no host
// staging, no copy engine).  The kernels are the ones muon_step launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/muon.h"
#include "api_internal.h"
#include "muon_internal.h"
#include "plan_host.h"

namespace muon {
namespace {

// One per device, resident from module load until the process ends.  Host
// code never passes its name to a kernel or a copy: the device address comes
// from hipGetSymbolAddress (scratch_base) and only that address is used.
__device__ __align__(256) char scratch[MUON_NOALLOC_SCRATCH_BYTES];

// What the scratch array of one device holds.
struct ScratchState {
  char* base = nullptr;            // device address of `scratch` on this device
  std::vector<int64_t> table_key;  // shapes whose tables are resident
  std::vector<PtrRecord> ptrs;     // pointers patched into those tables
  bool known = false;              // table_key / ptrs describe the device contents
  PlanTables tables;               // host image of the resident tables
  size_t table_off = 0;            // where the tables start in the scratch
};

std::map<int, ScratchState> g_scratch;

// Called with the device current, the first time a call runs on it.
int scratch_base(ScratchState& sc, char** out) {
  if (!sc.base) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MUON_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    sc.base = static_cast<char*>(ptr);
  }
  *out = sc.base;
  return MUON_OK;
}

// A host image to device memory through kernel arguments, in stream order.
int write_image(char* dst, const std::vector<char>& image, hipStream_t stream) {
  const size_t words = image.size() / 4;  // the image is a multiple of 256 bytes
  for (size_t w0 = 0; w0 < words; w0 += BLOB_WORDS) {
    BlobChunk c{};
    c.words = (int32_t)std::min<size_t>(BLOB_WORDS, words - w0);
    memcpy(c.w, image.data() + 4 * w0, 4 * (size_t)c.words);
    const hipError_t e = launch_blob_write(dst + 4 * w0, c, stream);
    if (e != hipSuccess) return fail_hip(e, "table write launch");
  }
  return MUON_OK;
}

int noalloc_entry(float* const* params, const float* const* grads, float* const* momentum, const muon_shape_t* shapes,
                  int n, float lr, float beta, int ns_steps, const float* coeffs, hipStream_t stream) {
  clear_error();
  int rc = validate_step(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, 0, nullptr);
  if (rc || n == 0) return rc;
  const size_t ws_need = workspace_bytes_of(shapes, n);
  if (ws_need > (size_t)MUON_NOALLOC_SCRATCH_BYTES)
    return fail(MUON_ENOMEM, "this call needs %zu bytes of workspace; the static scratch holds %zu", ws_need,
                (size_t)MUON_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  bool capturing = false;
  if ((rc = capture_status(stream, &capturing))) return rc;
  std::vector<PtrRecord> recs;
  make_ptr_records(MODE_STEP, shapes, n, params, grads, momentum, nullptr, nullptr, &recs);
  std::lock_guard<std::mutex> lock(api_mutex());
  ScratchState& sc = g_scratch[dev];
  char* base = nullptr;
  if ((rc = scratch_base(sc, &base))) return rc;
  std::vector<int64_t> key;
  key.reserve(2 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    key.push_back(shapes[i].rows);
    key.push_back(shapes[i].cols);
  }
  // The tables follow the workspace in the scratch.  They are rebuilt when
  // the shapes change, and written whenever the scratch is not known to hold
  // them (under capture always, so that a replay finds its own).
  if (!(sc.known && sc.table_key == key)) {
    PlanTables t;
    if ((rc = build_tables(MODE_STEP, shapes, n, base, 1, &t))) return rc;
    const size_t off = align_up(ws_need);
    if (off + t.image.size() > (size_t)MUON_NOALLOC_SCRATCH_BYTES)
      return fail(MUON_ENOMEM, "this call needs %zu bytes of workspace and tables; the static scratch holds %zu",
                  off + t.image.size(), (size_t)MUON_NOALLOC_SCRATCH_BYTES);
    sc.known = false;
    if ((rc = write_image(base + off, t.image, stream))) return rc;
    sc.tables = std::move(t);
    sc.table_off = off;
    sc.table_key = key;
    sc.ptrs.clear();
  } else if (capturing) {
    if ((rc = write_image(base + sc.table_off, sc.tables.image, stream))) return rc;
  }
  MatDesc* desc = reinterpret_cast<MatDesc*>(base + sc.table_off + sc.tables.o_desc);
  if (capturing || !sc.known || !same_records(sc.ptrs, recs)) {
    sc.known = false;
    if ((rc = patch_records(desc, recs, stream))) return rc;
    sc.ptrs = recs;
  }
  // after a capture the device holds whatever the last replay wrote
  sc.known = !capturing;
  return launch_sequence(MODE_STEP, tables_at(base + sc.table_off, sc.tables, 0, base), lr, beta, ns_steps, coeffs, 0,
                         stream);
}

}  // namespace
}  // namespace muon

extern "C" int muon_step_noalloc(float* const* params, const float* const* grads, float* const* momentum,
                                 const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
                                 const float* coeffs, hipStream_t stream) {
  return muon::noalloc_entry(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, stream);
}
