// Pieces of the C ABI's HIP side shared by its translation units: error
// text for HIP failures, stream-capture detection, the device addresses of a
// plan's tables and the launch sequence of one call.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "muon_internal.h"
#include "plan_host.h"

namespace muon {

int fail_hip(hipError_t e, const char* what);
int capture_status(hipStream_t stream, bool* capturing);

// Serialises every entry point's use of the library's host state.
std::mutex& api_mutex();

// Device addresses of one lane's tables (a table block laid out as t says,
// over the workspace ws).
struct Tables {
  MatDesc* desc;
  int32_t* mats;
  int32_t* fin;
  EwItem *mom, *cast, *apply;
  GemmItem *gram, *poly, *upd;
  RedItem* red;
  float* gram_part;
  bool small;
  bool fused;
  int gram_tile, poly_tile, upd_tile, gram_bm;  // TileKind of each GEMM, Gram tile edge
  const LaneTables* t;
};
Tables tables_at(char* block, const PlanTables& t, int lane, char* ws);

// Pointer records into the descriptors at desc, PATCH_MAX per launch.
int patch_records(MatDesc* desc, const std::vector<PtrRecord>& recs, hipStream_t stream);

// The kernel sequence of one lane of a call (the caller holds api_mutex()).
int launch_sequence(int mode, const Tables& v, float lr, float beta, int ns_steps, const float* coeffs, int stride,
                    hipStream_t stream);

}  // namespace muon
