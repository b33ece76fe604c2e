// Host side of the library that needs no GPU: argument validation, shape
// canonicalisation and workspace layout, the device table images (matrix
// descriptors and work lists), and the per-device plan cache.  Plain C++:
// built into libmuon.so and, with the host compiler alone, into a sanitizer
// build that exercises it against a fake device.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <list>
#include <memory>
#include <vector>

#include "../../include/muon.h"
#include "plan_types.h"

namespace muon {

// Thread-local error text of the last failing call (muon_last_error).
int fail(int code, const char* fmt, ...);
const char* last_error_text();
void clear_error();

// Canonical geometry of one matrix (m <= n, padded, workspace sizes).
struct Geometry {
  int32_t rows, cols, m, n, m_pad, n_pad, ld_x, ld_a, transposed, part_cnt;
  size_t x_bytes, a_bytes, part_bytes;
};
Geometry geometry_of(const muon_shape_t& s);

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

// Control region at the start of every workspace: one normalisation scale
// per matrix slot.
constexpr size_t kControlBytes = sizeof(float) * MUON_MAX_MATRICES;

// ---- validation (every check runs before any device call) ----
int check_shapes(const muon_shape_t* shapes, int n);
int check_coeffs(const float* coeffs, int ns_steps, int stride);
int validate_step(float* const* params, const float* const* grads, float* const* moms, const muon_shape_t* shapes,
                  int n, float lr, float beta, int ns_steps, const float* coeffs, int stride, uint16_t* const* upd);
int validate_ns(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n, int ns_steps,
                const float* coeffs, int stride);
int validate_adamw(float* const* params, const float* const* grads, float* const* u, float* const* v,
                   const int64_t* numels, const float* wd, int n, float lr, float beta1, float beta2, float eps,
                   int64_t step);
int validate_untie(const float* const src[3], float* const dst[3], int64_t rows, int64_t cols, int transpose);

// Workspace bytes of a call: control region, per-matrix iterates, A, B and
// norm partials, and the fp32 partial tiles of cut long-K Gram tiles.
size_t workspace_bytes_of(const muon_shape_t* shapes, int n);

enum Mode { MODE_STEP = 0, MODE_NS = 1 };

// Work lists of one lane: a group of matrices whose whole step runs as one
// launch sequence (on a stream of its own when a call has several lanes).
// fin: the matrices whose norm scale the finalisation kernel sums (more than
// NORM_FOLD_MAX partials; the cast sums the others itself).
struct LaneTables {
  size_t o_mats = 0, o_fin = 0, o_mom = 0, o_cast = 0, o_apply = 0, o_gram = 0, o_poly = 0, o_upd = 0, o_red = 0;
  int n_mats = 0, n_fin = 0, n_mom = 0, n_cast = 0, n_apply = 0, n_gram = 0, n_poly = 0, n_upd = 0, n_red = 0;
};

// Host image of a plan's device table block: descriptors (workspace pointers
// filled in, caller pointers left null) followed by each lane's matrix list
// and work lists.
struct PlanTables {
  std::vector<char> image;
  size_t o_desc = 0;
  int n_mat = 0;
  std::vector<LaneTables> lanes;
  size_t gram_part_off = 0;  // Gram partial tiles, offset in the workspace
  bool small = false;        // small-tile kernels (small_call)
  bool fused = false;        // small, and every m_pad is 256: poly and update in one launch
  int gram_tile = TILE_LARGE, poly_tile = TILE_LARGE, upd_tile = TILE_LARGE;  // TileKind of each GEMM
  int gram_bm = GRAM_BM;     // Gram tile edge (also of its partial tiles)
};

// A call is small when it has at most SMALL_MAX_UPD_TILES update tiles of
// UPD_BM x UPD_BN and no Gram K longer than SMALL_MAX_GRAM_SLICES slices: it
// then runs the small-tile kernels and never cuts Gram tiles.
bool small_call(const muon_shape_t* shapes, int n);

// The tile kind of each GEMM of a call (TileKind; see plan_types.h) and the
// Gram tile edge.
struct TileChoice {
  int gram = TILE_LARGE, poly = TILE_LARGE, upd = TILE_LARGE;
  int gram_bm = GRAM_BM;
};
TileChoice tile_choice(const muon_shape_t* shapes, int n);

// Lanes: matrices of one canonical shape always share a lane; shape groups
// are spread over at most max_lanes lanes, largest Newton-Schulz cost first
// onto the least loaded lane.  The long-K Gram split is decided over the
// whole call, so the lanes change only which launch a tile belongs to, never
// a result.
constexpr int kMaxLanes = 4;
constexpr int kDefaultLanes = 1;
std::vector<int> lane_of_matrices(const muon_shape_t* shapes, int n, int max_lanes);
int build_tables(int mode, const muon_shape_t* shapes, int n, char* ws_base, int max_lanes, PlanTables* out);

// The caller pointers of one call, one record per matrix (mat = index).
void make_ptr_records(int mode, const muon_shape_t* shapes, int n, float* const* params, const float* const* grads,
                      float* const* moms, uint16_t* const* upd, const uint16_t* const* xin,
                      std::vector<PtrRecord>* out);
bool same_records(const std::vector<PtrRecord>& a, const std::vector<PtrRecord>& b);

// The device operations the plan cache needs, in the caller's stream order.
class DeviceOps {
 public:
  virtual ~DeviceOps() {}
  // A device table block plus host staging of the same size.
  virtual int alloc_tables(size_t bytes, void** dev, void** host) = 0;
  virtual void free_tables(void* dev, void* host) = 0;
  // Enqueue image -> dev (through the block's own host staging).
  virtual int upload(void* dev, void* host, const void* image, size_t bytes) = 0;
  // Enqueue the pointer records into the descriptors at dev_desc.
  virtual int patch(void* dev_desc, const PtrRecord* recs, int count) = 0;
  virtual int alloc_workspace(size_t bytes, void** p) = 0;
  virtual void free_workspace(void* p) = 0;
  // Wait until the device has finished all work enqueued so far.
  virtual int sync_device() = 0;
};

// A cached plan: one set of shapes (and mode) on one workspace.  Its table
// block holds the descriptors and work lists; the caller pointers in the
// descriptors are patched in stream order whenever a call brings others.
struct Plan {
  std::vector<int64_t> key;
  PlanTables t;
  void* dev = nullptr;   // table block (device)
  void* host = nullptr;  // its host staging
  char* ws = nullptr;    // workspace the descriptors point into
  bool captured = false;  // used under graph capture: kept until release
  bool ptrs_known = false;
  std::vector<PtrRecord> ptrs;  // what an eager call last patched in

  template <typename T>
  T* at(size_t off) const { return reinterpret_cast<T*>(static_cast<char*>(dev) + off); }
  float* gram_part() const { return reinterpret_cast<float*>(ws + t.gram_part_off); }
};

struct CacheStats {
  int64_t plan_builds = 0, uploads = 0, patch_calls = 0, syncs = 0, evictions = 0, ws_allocs = 0;
};

// Per-device plan cache.  Plans are keyed on (mode, shapes, workspace), not
// on pointers.  A call under graph capture must find its plan and a large
// enough workspace already there (it allocates nothing); its plan is then
// kept, with its workspace, until release_all(), and every later eager call
// on it re-patches its pointers, since a replay writes the captured ones.
class PlanCache {
 public:
  static constexpr size_t kMaxPlans = 8;  // uncaptured plans kept (LRU)

  explicit PlanCache(DeviceOps* ops) : ops_(ops) {}
  ~PlanCache();
  PlanCache(const PlanCache&) = delete;
  PlanCache& operator=(const PlanCache&) = delete;

  int prepare(int mode, const muon_shape_t* shapes, int n, int max_lanes, const std::vector<PtrRecord>& recs,
              bool capturing, Plan** out);
  // Caller-owned workspace (nullptr / 0: back to library-owned).
  int set_workspace(void* p, size_t bytes);
  // Frees every plan and workspace (the caller has synchronised).
  void release_all();

  CacheStats stats;
  void* workspace() const { return ws_; }
  size_t workspace_bytes() const { return ws_bytes_; }
  size_t plan_count() const { return plans_.size(); }

 private:
  int acquire_workspace(size_t need, bool capturing);
  void drop_uncaptured_on(char* ws);
  void free_plan(Plan* p);

  DeviceOps* ops_;
  char* ws_ = nullptr;
  size_t ws_bytes_ = 0;
  bool ws_owned_ = false;
  std::vector<void*> retired_;  // owned workspaces still referenced by captured plans
  std::list<std::unique_ptr<Plan>> plans_;  // most recently used first
};

}  // namespace muon
