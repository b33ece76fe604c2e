// C ABI of the Muon step library: argument checks, the per-call plan (shape
// canonicalisation, padding, workspace layout, work lists), the per-device
// workspace and plan cache, and the launch sequence.  The operation itself is
// described in include/muon.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "muon_internal.h"

using namespace muon;

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(MUON_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Control region at the start of every workspace: one normalisation scale per
// matrix slot.
constexpr size_t kScaleBytes = sizeof(float) * MUON_MAX_MATRICES;
constexpr size_t kControlBytes = kScaleBytes;

struct Geometry {
  int32_t rows, cols, m, n, m_pad, n_pad, ld_x, ld_a, transposed, part_cnt;
  size_t x_bytes, a_bytes, part_bytes;
};

Geometry geometry_of(const muon_shape_t& s) {
  Geometry g{};
  g.rows = (int32_t)s.rows;
  g.cols = (int32_t)s.cols;
  g.transposed = s.rows > s.cols;
  g.m = (int32_t)std::min(s.rows, s.cols);
  g.n = (int32_t)std::max(s.rows, s.cols);
  g.m_pad = (int32_t)round_up(g.m, NS_PAD_M);
  g.n_pad = (int32_t)round_up(g.n, NS_PAD_N);
  g.part_cnt = (int32_t)((s.rows * s.cols + MOM_CHUNK - 1) / MOM_CHUNK);
  g.ld_x = g.n_pad + NS_LD_PAD;
  g.ld_a = g.m_pad + NS_LD_PAD;
  g.x_bytes = align_up((size_t)g.m_pad * g.ld_x * 2);
  // A and B carry NS_PAD_M spare rows: an update tile may hang over the last
  // rows and fetch (never store) up to UPD_BM - UPD_ROWU rows past m_pad.
  static_assert(UPD_BM - UPD_ROWU <= NS_PAD_M, "spare rows");
  g.a_bytes = align_up((size_t)(g.m_pad + NS_PAD_M) * g.ld_a * 2);
  g.part_bytes = align_up((size_t)g.part_cnt * sizeof(double));
  return g;
}

int check_shapes(const muon_shape_t* shapes, int n) {
  if (n < 0 || n > MUON_MAX_MATRICES) return fail(MUON_EINVAL, "n = %d outside [0, %d]", n, MUON_MAX_MATRICES);
  if (n > 0 && !shapes) return fail(MUON_EINVAL, "shapes is NULL");
  for (int i = 0; i < n; ++i) {
    const int64_t r = shapes[i].rows, c = shapes[i].cols;
    if (r < 1 || c < 1) return fail(MUON_EINVAL, "matrix %d: shape %lld x %lld (both must be >= 1)", i, (long long)r, (long long)c);
    if (r > (int64_t)INT32_MAX || c > (int64_t)INT32_MAX || r * c >= ((int64_t)1 << 31))
      return fail(MUON_EINVAL, "matrix %d: shape %lld x %lld has 2^31 or more elements", i, (long long)r, (long long)c);
    const Geometry g = geometry_of(shapes[i]);
    if ((int64_t)g.m_pad * g.ld_x >= ((int64_t)1 << 31) || (int64_t)(g.m_pad + NS_PAD_M) * g.ld_a >= ((int64_t)1 << 31))
      return fail(MUON_EINVAL, "matrix %d: padded shape too large", i);
  }
  return MUON_OK;
}

// Long-K Gram split of a call (GRAM_SPLIT_MIN): the chunk length in K
// slices, 0 when no tile is cut, and the fp32 partial tiles it needs.
struct GramSplit {
  int64_t chunk = 0;
  int64_t slots = 0;
};

// K slices of a Gram tile: the product runs to the true n (the padding is zero).
int64_t gram_slices(const Geometry& g) { return ((int64_t)g.n + 63) / 64; }
int64_t gram_tiles(const Geometry& g) {
  const int64_t t = g.m_pad / GRAM_BM;
  return t * (t + 1) / 2;
}
int64_t gram_chunks(int64_t slices, int64_t chunk) {
  return (chunk && slices > chunk) ? (slices + chunk - 1) / chunk : 1;
}

GramSplit gram_split_of(const muon_shape_t* shapes, int n) {
  GramSplit sp;
  int64_t total = 0, longest = 0;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    total += gram_tiles(g) * gram_slices(g);
    longest = std::max(longest, gram_slices(g));
  }
  const int64_t share = std::max<int64_t>(GRAM_SPLIT_MIN, (total + NS_CUS - 1) / NS_CUS);
  if (longest <= 2 * share) return sp;
  sp.chunk = share;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    const int64_t nc = gram_chunks(gram_slices(g), sp.chunk);
    if (nc > 1) sp.slots += gram_tiles(g) * nc;
  }
  return sp;
}

size_t workspace_bytes_of(const muon_shape_t* shapes, int n) {
  size_t total = kControlBytes;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    total += 2 * g.x_bytes + 2 * g.a_bytes + g.part_bytes;
  }
  total += align_up((size_t)gram_split_of(shapes, n).slots * GRAM_BM * GRAM_BM * sizeof(float));
  return total;
}

// Coefficients: one {a, b, c} for every iteration (stride 0, always required),
// or a schedule of ns_steps triples (stride 3; may be NULL when ns_steps = 0).
int check_coeffs(const float* coeffs, int ns_steps, int stride) {
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS)
    return fail(MUON_EINVAL, "ns_steps = %d outside [0, %d]", ns_steps, MUON_MAX_NS_STEPS);
  const int count = stride ? 3 * ns_steps : 3;
  if (count == 0) return MUON_OK;
  if (!coeffs) return fail(MUON_EINVAL, "coeffs is NULL");
  for (int k = 0; k < count; ++k)
    if (!std::isfinite(coeffs[k])) return fail(MUON_EINVAL, "coeffs[%d] is not finite", k);
  return MUON_OK;
}

struct Range {
  uintptr_t lo, hi;
  int mat;
  const char* what;
};

// Every listed array must be non-null, aligned, and disjoint from the others.
int check_ranges(std::vector<Range>& v) {
  std::sort(v.begin(), v.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < v.size(); ++k)
    if (v[k].lo < v[k - 1].hi)
      return fail(MUON_EINVAL, "%s of matrix %d overlaps %s of matrix %d", v[k].what, v[k].mat,
                  v[k - 1].what, v[k - 1].mat);
  return MUON_OK;
}

// ---------------------------------------------------------------- plans ----

enum Mode { MODE_STEP = 0, MODE_NS = 1 };

struct Plan {
  std::vector<uintptr_t> key;
  void* dev = nullptr;   // descriptors + work lists (device)
  void* host = nullptr;  // pinned staging of the same bytes
  size_t bytes = 0;
  MatDesc* d_desc = nullptr;
  EwItem* d_mom = nullptr;
  EwItem* d_cast = nullptr;
  EwItem* d_apply = nullptr;
  GemmItem* d_gram = nullptr;
  GemmItem* d_poly = nullptr;
  GemmItem* d_upd = nullptr;
  RedItem* d_red = nullptr;
  float* gram_part = nullptr;  // fp32 partial tiles of split Gram tiles (workspace)
  int n_mom = 0, n_cast = 0, n_apply = 0, n_gram = 0, n_poly = 0, n_upd = 0, n_red = 0;
  ~Plan() {
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
  }
};

// AdamW work list: tensor descriptors and chunk items, cached per pointer set.
struct AdamPlan {
  std::vector<uintptr_t> key;
  void* dev = nullptr;
  void* host = nullptr;
  AdamDesc* d_desc = nullptr;
  EwItem* d_items = nullptr;
  int n_items = 0;
  ~AdamPlan() {
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
  }
};

struct DeviceState {
  void* ws = nullptr;       // workspace in use (owned or caller's)
  size_t ws_bytes = 0;
  bool ws_owned = false;
  std::list<std::unique_ptr<Plan>> plans;  // most recent first
  std::list<std::unique_ptr<AdamPlan>> adam_plans;  // most recent first
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;
constexpr size_t kMaxPlans = 8;

// Timing of one kernel family (muon_timing_enable).
int g_time_kind = -1;
std::vector<hipEvent_t> g_ev;  // start, end pairs
size_t g_ev_used = 0;

int clear_plans(DeviceState& st) {
  st.plans.clear();
  return MUON_OK;
}

int acquire_workspace(DeviceState& st, size_t need, hipStream_t stream) {
  if (st.ws && st.ws_bytes >= need) return MUON_OK;
  if (st.ws && !st.ws_owned)
    return fail(MUON_ENOMEM, "caller workspace has %zu bytes, this call needs %zu", st.ws_bytes, need);
  const char* inject = getenv("MUON_TEST_FAIL_ALLOC");
  if (inject && inject[0] == '1') return fail(MUON_ENOMEM, "workspace allocation of %zu bytes failed (injected)", need);
  // Growing: wait for work that may still use the old buffer, then replace it.
  hipError_t e;
  if (st.ws) {
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
    (void)hipFree(st.ws);
    st.ws = nullptr;
    st.ws_bytes = 0;
    clear_plans(st);
  }
  size_t want = std::max(need, (size_t)(need * 1.25));
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    want = need;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MUON_ENOMEM, "hipMalloc of %zu workspace bytes failed: %s", want, hipGetErrorString(e));
    }
  }
  st.ws = p;
  st.ws_bytes = want;
  st.ws_owned = true;
  return MUON_OK;
}

// Workgroup w of a launch runs on XCD w % kXcds, and each XCD has its own L2.
// Cut the locality-ordered tile sequence into kXcds contiguous runs of about
// equal cost and interleave them, so that each XCD works through one run and
// its concurrently resident tiles share operands in that XCD's L2.  Within a
// run, tiles are dispatched longest first (stable, so tiles of equal cost
// keep their locality order): the short ones then fill the gaps at the end
// instead of a long tile starting last.  Runs of unequal length are padded
// with empty items (mat = -1) that exit at once.
constexpr int kXcds = 8;

std::vector<GemmItem> xcd_interleave(const std::vector<GemmItem>& seq, const std::vector<int64_t>& cost) {
  int64_t total = 0;
  for (int64_t c : cost) total += c;
  std::vector<std::vector<std::pair<int64_t, GemmItem>>> run(kXcds);
  int64_t acc = 0;
  int x = 0;
  for (size_t k = 0; k < seq.size(); ++k) {
    while (x < kXcds - 1 && acc >= total * (x + 1) / kXcds) ++x;
    run[x].push_back({cost[k], seq[k]});
    acc += cost[k];
  }
  size_t len = 0;
  for (auto& r : run) {
    std::stable_sort(r.begin(), r.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
    len = std::max(len, r.size());
  }
  std::vector<GemmItem> out(len * kXcds, GemmItem{-1, 0, 0, 0, 0, -1});
  for (int r = 0; r < kXcds; ++r)
    for (size_t k = 0; k < run[r].size(); ++k) out[k * kXcds + r] = run[r][k].second;
  return out;
}

template <typename T>
T* carve(char*& cur, size_t count) {
  T* p = reinterpret_cast<T*>(cur);
  cur += align_up(count * sizeof(T));
  return p;
}

// Build (or fetch) the plan for this call.  Descriptors point into the
// current workspace; the cache is dropped whenever the workspace changes.
int get_plan(DeviceState& st, int mode, int n, const muon_shape_t* shapes, float* const* params,
             const float* const* grads, float* const* moms, uint16_t* const* upd, const uint16_t* const* xin,
             hipStream_t stream, Plan** out) {
  std::vector<uintptr_t> key;
  key.reserve(8 + 6 * (size_t)n);
  key.push_back((uintptr_t)mode);
  key.push_back((uintptr_t)n);
  key.push_back((uintptr_t)st.ws);
  for (int i = 0; i < n; ++i) {
    key.push_back((uintptr_t)shapes[i].rows);
    key.push_back((uintptr_t)shapes[i].cols);
    key.push_back(params ? (uintptr_t)params[i] : 0);
    key.push_back(grads ? (uintptr_t)grads[i] : 0);
    key.push_back(moms ? (uintptr_t)moms[i] : (xin ? (uintptr_t)xin[i] : 0));
    key.push_back(upd ? (uintptr_t)upd[i] : 0);
  }
  for (auto it = st.plans.begin(); it != st.plans.end(); ++it) {
    if ((*it)->key == key) {
      if (it != st.plans.begin()) st.plans.splice(st.plans.begin(), st.plans, it);
      *out = st.plans.front().get();
      return MUON_OK;
    }
  }

  auto plan = std::make_unique<Plan>();
  plan->key = std::move(key);
  std::vector<MatDesc> desc(n);
  std::vector<EwItem> mom, cast, apply;
  std::vector<GemmItem> gram, poly, updl;
  char* cur = static_cast<char*>(st.ws);
  float* scales = reinterpret_cast<float*>(cur);
  cur += kControlBytes;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    MatDesc& d = desc[i];
    memset(&d, 0, sizeof d);
    d.W = params ? params[i] : nullptr;
    d.G = grads ? grads[i] : nullptr;
    d.M = moms ? moms[i] : nullptr;
    d.upd = upd ? upd[i] : nullptr;
    d.xin = xin ? xin[i] : nullptr;
    d.X[0] = carve<uint16_t>(cur, g.x_bytes / 2);
    d.X[1] = carve<uint16_t>(cur, g.x_bytes / 2);
    d.A = carve<uint16_t>(cur, g.a_bytes / 2);
    d.B = carve<uint16_t>(cur, g.a_bytes / 2);
    d.part = carve<double>(cur, g.part_bytes / sizeof(double));
    d.scale = scales + i;
    d.rows = g.rows;
    d.cols = g.cols;
    d.m = g.m;
    d.n = g.n;
    d.m_pad = g.m_pad;
    d.n_pad = g.n_pad;
    d.ld_x = g.ld_x;
    d.ld_a = g.ld_a;
    d.transposed = g.transposed;
    d.part_cnt = g.part_cnt;
    if (mode == MODE_STEP) {
      const bool aligned = ((uintptr_t)d.W % 16 == 0) && ((uintptr_t)d.G % 16 == 0) && ((uintptr_t)d.M % 16 == 0);
      d.vec4 = aligned && (g.cols % 4 == 0);
      for (int c = 0; c < g.part_cnt; ++c) mom.push_back({i, c});
    } else {
      d.vec4 = ((uintptr_t)d.xin % 8 == 0) && (g.cols % 4 == 0);
    }
    const int ct = (g.m_pad / CAST_TILE) * (g.n_pad / CAST_TILE);
    for (int t = 0; t < ct; ++t) cast.push_back({i, t});
    const int at = ((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE);
    for (int t = 0; t < at; ++t) apply.push_back({i, t});
  }
  // The cast re-reads what the momentum pass just streamed: walking it
  // backwards starts with the lines most likely still in the memory-side
  // cache.
  std::reverse(cast.begin(), cast.end());
  // Partial tiles of split Gram tiles follow the matrices' buffers.
  const GramSplit split = gram_split_of(shapes, n);
  plan->gram_part = carve<float>(cur, (size_t)split.slots * GRAM_BM * GRAM_BM);
  // GEMM tiles.  Per matrix in an order that reuses operands (update: all row
  // tiles of one column block in a row, sharing that block of X; symmetric
  // phases: upper-triangle tiles row by row), then spread over the XCDs.
  // Gram and poly tiles differ in size (256 and 128); a long-K Gram tile may
  // be cut into K chunks, each its own item, summed by the reduce pass.
  std::vector<GemmItem> gram_seq, poly_seq, upd_seq;
  std::vector<RedItem> red;
  std::vector<int64_t> gram_cost, upd_cost;
  int32_t slot = 0;
  for (int i = 0; i < n; ++i) {
    const int tg = desc[i].m_pad / GRAM_BM, tm = desc[i].m_pad / SYM_BM, tn = desc[i].n_pad / UPD_BN;
    const int64_t ks = ((int64_t)desc[i].n + 63) / 64;            // Gram K slices
    const int32_t kp = (int32_t)(((int64_t)desc[i].m + 63) / 64);      // poly K slices
    const int32_t ku = (int32_t)(2 * (((int64_t)desc[i].m + 127) / 128));  // update: even, see the kernel
    const int64_t nc = gram_chunks(ks, split.chunk);
    for (int ti = 0; ti < tg; ++ti)
      for (int tj = ti; tj < tg; ++tj) {
        if (nc == 1) {
          gram_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, (int32_t)ks, -1});
          gram_cost.push_back(ks);
          continue;
        }
        for (int64_t c = 0; c < nc; ++c) {
          const int64_t a = ks * c / nc, b = ks * (c + 1) / nc;
          gram_seq.push_back({i, (int16_t)ti, (int16_t)tj, (int32_t)a, (int32_t)(b - a), slot + (int32_t)c});
          gram_cost.push_back(b - a);
        }
        constexpr int SUB = GRAM_BM / RED_TILE;
        for (int bi = 0; bi < SUB; ++bi)
          for (int bj = 0; bj < SUB; ++bj)
            if (ti != tj || bi <= bj) red.push_back({i, (int16_t)ti, (int16_t)tj, slot, (int16_t)nc, (int8_t)bi, (int8_t)bj});
        slot += (int32_t)nc;
      }
    for (int ti = 0; ti < tm; ++ti)
      for (int tj = ti; tj < tm; ++tj) poly_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, kp, -1});
    for (int tj = 0; tj < tn; ++tj)
      for (int ti = 0; ti < desc[i].m_pad / UPD_ROWU; ti += UPD_BM / UPD_ROWU) {
        upd_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, ku, -1});
        upd_cost.push_back(ku);
      }
  }
  if (slot != split.slots) return fail(MUON_EINVAL, "internal: %d Gram partial tiles planned, %lld sized", slot, (long long)split.slots);
  std::vector<int64_t> poly_cost(poly_seq.size());
  for (size_t k = 0; k < poly_seq.size(); ++k) poly_cost[k] = poly_seq[k].kn;
  gram = xcd_interleave(gram_seq, gram_cost);
  poly = xcd_interleave(poly_seq, poly_cost);
  updl = xcd_interleave(upd_seq, upd_cost);

  size_t off = 0;
  auto place = [&](size_t bytes) { const size_t o = off; off += align_up(bytes); return o; };
  const size_t o_desc = place(sizeof(MatDesc) * n);
  const size_t o_mom = place(sizeof(EwItem) * mom.size());
  const size_t o_cast = place(sizeof(EwItem) * cast.size());
  const size_t o_apply = place(sizeof(EwItem) * apply.size());
  const size_t o_gram = place(sizeof(GemmItem) * gram.size());
  const size_t o_poly = place(sizeof(GemmItem) * poly.size());
  const size_t o_upd = place(sizeof(GemmItem) * updl.size());
  const size_t o_red = place(sizeof(RedItem) * red.size());
  plan->bytes = std::max<size_t>(off, kAlign);
  hipError_t e;
  if ((e = hipHostMalloc(&plan->host, plan->bytes, hipHostMallocDefault)) != hipSuccess) {
    plan->host = nullptr;
    return fail(MUON_ENOMEM, "hipHostMalloc of %zu plan bytes failed: %s", plan->bytes, hipGetErrorString(e));
  }
  if ((e = hipMalloc(&plan->dev, plan->bytes)) != hipSuccess) {
    plan->dev = nullptr;
    (void)hipGetLastError();
    return fail(MUON_ENOMEM, "hipMalloc of %zu plan bytes failed: %s", plan->bytes, hipGetErrorString(e));
  }
  char* h = static_cast<char*>(plan->host);
  memcpy(h + o_desc, desc.data(), sizeof(MatDesc) * n);
  memcpy(h + o_mom, mom.data(), sizeof(EwItem) * mom.size());
  memcpy(h + o_cast, cast.data(), sizeof(EwItem) * cast.size());
  memcpy(h + o_apply, apply.data(), sizeof(EwItem) * apply.size());
  memcpy(h + o_gram, gram.data(), sizeof(GemmItem) * gram.size());
  memcpy(h + o_poly, poly.data(), sizeof(GemmItem) * poly.size());
  memcpy(h + o_upd, updl.data(), sizeof(GemmItem) * updl.size());
  memcpy(h + o_red, red.data(), sizeof(RedItem) * red.size());
  if ((e = hipMemcpyAsync(plan->dev, plan->host, plan->bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
    return fail_hip(e, "hipMemcpyAsync(plan)");
  // One-time wait so the plan is usable from any stream afterwards.
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize(plan)");
  char* dv = static_cast<char*>(plan->dev);
  plan->d_desc = reinterpret_cast<MatDesc*>(dv + o_desc);
  plan->d_mom = reinterpret_cast<EwItem*>(dv + o_mom);
  plan->d_cast = reinterpret_cast<EwItem*>(dv + o_cast);
  plan->d_apply = reinterpret_cast<EwItem*>(dv + o_apply);
  plan->d_gram = reinterpret_cast<GemmItem*>(dv + o_gram);
  plan->d_poly = reinterpret_cast<GemmItem*>(dv + o_poly);
  plan->d_upd = reinterpret_cast<GemmItem*>(dv + o_upd);
  plan->d_red = reinterpret_cast<RedItem*>(dv + o_red);
  plan->n_mom = (int)mom.size();
  plan->n_cast = (int)cast.size();
  plan->n_apply = (int)apply.size();
  plan->n_gram = (int)gram.size();
  plan->n_poly = (int)poly.size();
  plan->n_upd = (int)updl.size();
  plan->n_red = (int)red.size();
  st.plans.push_front(std::move(plan));
  while (st.plans.size() > kMaxPlans) st.plans.pop_back();
  *out = st.plans.front().get();
  return MUON_OK;
}

// Launch wrapper: brackets the launch with events when its family is timed.
template <typename F>
int timed(int kind, hipStream_t stream, F&& launch, const char* what) {
  const bool on = (g_time_kind == kind);
  hipError_t e;
  if (on) {
    if (g_ev_used + 2 > g_ev.size()) {
      for (int k = 0; k < 2; ++k) {
        hipEvent_t ev;
        if ((e = hipEventCreate(&ev)) != hipSuccess) return fail_hip(e, "hipEventCreate");
        g_ev.push_back(ev);
      }
    }
    if ((e = hipEventRecord(g_ev[g_ev_used], stream)) != hipSuccess) return fail_hip(e, "hipEventRecord");
  }
  if ((e = launch()) != hipSuccess) return fail_hip(e, what);
  if (on) {
    if ((e = hipEventRecord(g_ev[g_ev_used + 1], stream)) != hipSuccess) return fail_hip(e, "hipEventRecord");
    g_ev_used += 2;
  }
  return MUON_OK;
}

int run(int mode, float* const* params, const float* const* grads, float* const* moms,
        uint16_t* const* upd, const uint16_t* const* xin, const muon_shape_t* shapes, int n, float lr,
        float beta, int ns_steps, const float* coeffs, int stride, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  int rc = acquire_workspace(st, workspace_bytes_of(shapes, n), stream);
  if (rc) return rc;
  Plan* p = nullptr;
  if ((rc = get_plan(st, mode, n, shapes, params, grads, moms, upd, xin, stream, &p))) return rc;
  if (mode == MODE_STEP) {
    rc = timed(MUON_KERNEL_MOMENTUM, stream, [&] { return launch_momentum(p->d_desc, p->d_mom, p->n_mom, n, beta, stream); },
               "momentum kernel launch");
    if (rc) return rc;
  }
  rc = timed(MUON_KERNEL_CAST, stream,
             [&] { return launch_cast(p->d_desc, p->d_cast, p->n_cast, beta, mode == MODE_NS, stream); },
             "cast kernel launch");
  if (rc) return rc;
  for (int k = 0; k < ns_steps; ++k) {
    const int src = k & 1;
    const float* ck = coeffs + (size_t)k * stride;  // iteration k's a, b, c
    const float ca = ck[0], cb = ck[1], cc = ck[2];
    rc = timed(MUON_KERNEL_GRAM, stream,
               [&] {
                 const hipError_t e = launch_gemm(GEMM_GRAM, p->d_desc, p->d_gram, p->n_gram, src, ca, cb, cc,
                                                  p->gram_part, stream);
                 return e != hipSuccess ? e : launch_gram_reduce(p->d_desc, p->d_red, p->n_red, p->gram_part, stream);
               },
               "gram kernel launch");
    if (rc) return rc;
    rc = timed(MUON_KERNEL_POLY, stream,
               [&] { return launch_gemm(GEMM_POLY, p->d_desc, p->d_poly, p->n_poly, src, ca, cb, cc, nullptr, stream); },
               "poly kernel launch");
    if (rc) return rc;
    rc = timed(MUON_KERNEL_UPDATE, stream,
               [&] { return launch_gemm(GEMM_UPDATE, p->d_desc, p->d_upd, p->n_upd, src, ca, cb, cc, nullptr, stream); },
               "update kernel launch");
    if (rc) return rc;
  }
  rc = timed(MUON_KERNEL_APPLY, stream,
             [&] { return launch_apply(p->d_desc, p->d_apply, p->n_apply, lr, ns_steps & 1, mode == MODE_STEP, stream); },
             "apply kernel launch");
  return rc;
}

int validate_step(float* const* params, const float* const* grads, float* const* moms, const muon_shape_t* shapes,
                  int n, float lr, float beta, int ns_steps, const float* coeffs, int stride, uint16_t* const* upd) {
  int rc = check_shapes(shapes, n);
  if (rc) return rc;
  if (!params || !grads || !moms) return fail(MUON_EINVAL, "params, grads and momentum arrays must not be NULL");
  if (!std::isfinite(lr)) return fail(MUON_EINVAL, "lr is not finite");
  if (!std::isfinite(beta) || beta < 0.0f || beta >= 1.0f) return fail(MUON_EINVAL, "beta = %g outside [0, 1)", (double)beta);
  if ((rc = check_coeffs(coeffs, ns_steps, stride))) return rc;
  std::vector<Range> r;
  r.reserve(4 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    const size_t fb = (size_t)shapes[i].rows * shapes[i].cols * sizeof(float);
    const void* ptrs[3] = {params[i], grads[i], moms[i]};
    const char* names[3] = {"params", "grads", "momentum"};
    for (int k = 0; k < 3; ++k) {
      if (!ptrs[k]) return fail(MUON_EINVAL, "%s[%d] is NULL", names[k], i);
      if ((uintptr_t)ptrs[k] % 4) return fail(MUON_EINVAL, "%s[%d] is not 4-byte aligned", names[k], i);
      r.push_back({(uintptr_t)ptrs[k], (uintptr_t)ptrs[k] + fb, i, names[k]});
    }
    if (upd && upd[i]) {
      if ((uintptr_t)upd[i] % 2) return fail(MUON_EINVAL, "updates[%d] is not 2-byte aligned", i);
      r.push_back({(uintptr_t)upd[i], (uintptr_t)upd[i] + fb / 2, i, "updates"});
    }
  }
  return check_ranges(r);
}

int step_entry(float* const* params, const float* const* grads, float* const* momentum, const muon_shape_t* shapes,
               int n, float lr, float beta, int ns_steps, const float* coeffs, int stride, uint16_t* const* updates,
               hipStream_t stream) {
  g_error.clear();
  int rc = validate_step(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, stride, updates);
  if (rc || n == 0) return rc;
  return run(MODE_STEP, params, grads, momentum, updates, nullptr, shapes, n, lr, beta, ns_steps, coeffs, stride,
             stream);
}

int ns_entry(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n, int ns_steps,
             const float* coeffs, int stride, hipStream_t stream) {
  g_error.clear();
  int rc = check_shapes(shapes, n);
  if (rc) return rc;
  if (!x || !out) return fail(MUON_EINVAL, "x and out arrays must not be NULL");
  if ((rc = check_coeffs(coeffs, ns_steps, stride))) return rc;
  std::vector<Range> r;
  for (int i = 0; i < n; ++i) {
    if (!x[i] || !out[i]) return fail(MUON_EINVAL, "x[%d] or out[%d] is NULL", i, i);
    if ((uintptr_t)x[i] % 2 || (uintptr_t)out[i] % 2) return fail(MUON_EINVAL, "x[%d] or out[%d] is not 2-byte aligned", i, i);
    const size_t b = (size_t)shapes[i].rows * shapes[i].cols * 2;
    r.push_back({(uintptr_t)out[i], (uintptr_t)out[i] + b, i, "out"});
    if (x[i] != out[i]) r.push_back({(uintptr_t)x[i], (uintptr_t)x[i] + b, i, "x"});
  }
  if ((rc = check_ranges(r))) return rc;
  if (n == 0) return MUON_OK;
  return run(MODE_NS, nullptr, nullptr, nullptr, out, x, shapes, n, 0.0f, 0.0f, ns_steps, coeffs, stride, stream);
}

// ---------------------------------------------------------------- AdamW ----

// wd[i] is a tensor's own lambda, baked into the plan, unless shared[i] is
// set: then the call's shared lambda (a kernel argument) applies.  The shared
// lambda can change from call to call (a weight-decay schedule) without a new
// plan.
int get_adam_plan(DeviceState& st, int n, float* const* params, const float* const* grads, float* const* u,
                  float* const* v, const int64_t* numels, const float* wd, const int* shared, hipStream_t stream,
                  AdamPlan** out) {
  std::vector<uintptr_t> key;
  key.reserve(1 + 7 * (size_t)n);
  key.push_back((uintptr_t)n);
  for (int i = 0; i < n; ++i) {
    uint32_t wbits = 0;
    memcpy(&wbits, &wd[i], sizeof wbits);
    key.push_back((uintptr_t)params[i]);
    key.push_back((uintptr_t)grads[i]);
    key.push_back((uintptr_t)u[i]);
    key.push_back((uintptr_t)v[i]);
    key.push_back((uintptr_t)numels[i]);
    key.push_back((uintptr_t)shared[i]);
    key.push_back(shared[i] ? 0 : (uintptr_t)wbits);
  }
  for (auto it = st.adam_plans.begin(); it != st.adam_plans.end(); ++it) {
    if ((*it)->key == key) {
      if (it != st.adam_plans.begin()) st.adam_plans.splice(st.adam_plans.begin(), st.adam_plans, it);
      *out = st.adam_plans.front().get();
      return MUON_OK;
    }
  }
  auto plan = std::make_unique<AdamPlan>();
  plan->key = std::move(key);
  std::vector<AdamDesc> desc(n);
  std::vector<EwItem> items;
  for (int i = 0; i < n; ++i) {
    AdamDesc& d = desc[i];
    memset(&d, 0, sizeof d);
    d.p = params[i];
    d.g = grads[i];
    d.u = u[i];
    d.v = v[i];
    d.numel = numels[i];
    d.wd = shared[i] ? 0.0f : wd[i];
    d.wd_shared = shared[i];
    d.vec4 = ((uintptr_t)d.p % 16 == 0) && ((uintptr_t)d.g % 16 == 0) && ((uintptr_t)d.u % 16 == 0) &&
             ((uintptr_t)d.v % 16 == 0);
    const int64_t chunks = (numels[i] + ADAM_CHUNK - 1) / ADAM_CHUNK;
    for (int64_t c = 0; c < chunks; ++c) items.push_back({i, (int32_t)c});
  }
  if (items.size() > (size_t)INT32_MAX) return fail(MUON_EINVAL, "AdamW call of %zu chunks is too large", items.size());
  const size_t o_desc = 0;
  const size_t o_items = align_up(sizeof(AdamDesc) * n);
  const size_t bytes = std::max<size_t>(o_items + align_up(sizeof(EwItem) * items.size()), kAlign);
  hipError_t e;
  if ((e = hipHostMalloc(&plan->host, bytes, hipHostMallocDefault)) != hipSuccess) {
    plan->host = nullptr;
    return fail(MUON_ENOMEM, "hipHostMalloc of %zu plan bytes failed: %s", bytes, hipGetErrorString(e));
  }
  if ((e = hipMalloc(&plan->dev, bytes)) != hipSuccess) {
    plan->dev = nullptr;
    (void)hipGetLastError();
    return fail(MUON_ENOMEM, "hipMalloc of %zu plan bytes failed: %s", bytes, hipGetErrorString(e));
  }
  char* h = static_cast<char*>(plan->host);
  memcpy(h + o_desc, desc.data(), sizeof(AdamDesc) * n);
  memcpy(h + o_items, items.data(), sizeof(EwItem) * items.size());
  if ((e = hipMemcpyAsync(plan->dev, plan->host, bytes, hipMemcpyHostToDevice, stream)) != hipSuccess)
    return fail_hip(e, "hipMemcpyAsync(adamw plan)");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return fail_hip(e, "hipStreamSynchronize(adamw plan)");
  plan->d_desc = reinterpret_cast<AdamDesc*>(static_cast<char*>(plan->dev) + o_desc);
  plan->d_items = reinterpret_cast<EwItem*>(static_cast<char*>(plan->dev) + o_items);
  plan->n_items = (int)items.size();
  st.adam_plans.push_front(std::move(plan));
  while (st.adam_plans.size() > kMaxPlans) st.adam_plans.pop_back();
  *out = st.adam_plans.front().get();
  return MUON_OK;
}

int validate_adamw(float* const* params, const float* const* grads, float* const* u, float* const* v,
                   const int64_t* numels, const float* wd, int n, float lr, float beta1, float beta2, float eps,
                   int64_t step) {
  if (n < 0 || n > MUON_ADAMW_MAX_TENSORS)
    return fail(MUON_EINVAL, "n = %d outside [0, %d]", n, MUON_ADAMW_MAX_TENSORS);
  if (n > 0 && (!params || !grads || !u || !v || !numels))
    return fail(MUON_EINVAL, "params, grads, exp_avg, exp_avg_sq and numels arrays must not be NULL");
  if (!std::isfinite(lr)) return fail(MUON_EINVAL, "lr is not finite");
  if (!std::isfinite(beta1) || beta1 < 0.0f || beta1 >= 1.0f) return fail(MUON_EINVAL, "beta1 = %g outside [0, 1)", (double)beta1);
  if (!std::isfinite(beta2) || beta2 < 0.0f || beta2 >= 1.0f) return fail(MUON_EINVAL, "beta2 = %g outside [0, 1)", (double)beta2);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(MUON_EINVAL, "eps = %g is not finite and >= 0", (double)eps);
  if (step < 1) return fail(MUON_EINVAL, "step = %lld: the first step is 1", (long long)step);
  std::vector<Range> r;
  r.reserve(4 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    if (numels[i] < 0) return fail(MUON_EINVAL, "numels[%d] = %lld is negative", i, (long long)numels[i]);
    if (wd && (!std::isfinite(wd[i]) || wd[i] < 0.0f))
      return fail(MUON_EINVAL, "weight_decay[%d] = %g is not finite and >= 0", i, (double)wd[i]);
    if (numels[i] == 0) continue;
    if (numels[i] > (int64_t)1 << 40) return fail(MUON_EINVAL, "numels[%d] = %lld is too large", i, (long long)numels[i]);
    const size_t fb = (size_t)numels[i] * sizeof(float);
    const void* ptrs[4] = {params[i], grads[i], u[i], v[i]};
    const char* names[4] = {"params", "grads", "exp_avg", "exp_avg_sq"};
    for (int k = 0; k < 4; ++k) {
      if (!ptrs[k]) return fail(MUON_EINVAL, "%s[%d] is NULL", names[k], i);
      if ((uintptr_t)ptrs[k] % 4) return fail(MUON_EINVAL, "%s[%d] is not 4-byte aligned", names[k], i);
      r.push_back({(uintptr_t)ptrs[k], (uintptr_t)ptrs[k] + fb, i, names[k]});
    }
  }
  return check_ranges(r);
}

int adamw_entry(float* const* params, const float* const* grads, float* const* u, float* const* v,
                const int64_t* numels, const float* wd, int n, float lr, float beta1, float beta2, float eps,
                int64_t step, hipStream_t stream) {
  g_error.clear();
  int rc = validate_adamw(params, grads, u, v, numels, wd, n, lr, beta1, beta2, eps, step);
  if (rc) return rc;
  // tensors with elements; empty ones are dropped before planning
  std::vector<float*> P, U, V;
  std::vector<const float*> G;
  std::vector<int64_t> N;
  std::vector<float> W;
  for (int i = 0; i < n; ++i) {
    if (numels[i] == 0) continue;
    P.push_back(params[i]);
    G.push_back(grads[i]);
    U.push_back(u[i]);
    V.push_back(v[i]);
    N.push_back(numels[i]);
    W.push_back(wd ? wd[i] : 0.0f);
  }
  if (P.empty()) return MUON_OK;
  // The first non-zero lambda is the call's shared one; every tensor that
  // uses it takes it from the kernel arguments.
  std::vector<int> S(W.size(), 0);
  float shared_wd = 0.0f;
  for (float w : W)
    if (w != 0.0f) {
      shared_wd = w;
      break;
    }
  for (size_t i = 0; i < W.size(); ++i) S[i] = (W[i] != 0.0f && W[i] == shared_wd) ? 1 : 0;
  AdamConst c{};
  c.wd_shared = shared_wd;
  c.lr = lr;
  c.beta1 = beta1;
  c.beta2 = beta2;
  c.eps = eps;
  c.omb1 = (float)(1.0 - (double)beta1);
  c.omb2 = (float)(1.0 - (double)beta2);
  c.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  c.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  AdamPlan* p = nullptr;
  if ((rc = get_adam_plan(st, (int)P.size(), P.data(), G.data(), U.data(), V.data(), N.data(), W.data(), S.data(), stream,
                          &p)))
    return rc;
  return timed(MUON_KERNEL_ADAMW, stream, [&] { return launch_adamw(p->d_desc, p->d_items, p->n_items, c, stream); },
               "adamw kernel launch");
}

int untie_entry(const float* const src[3], float* const dst[3], int64_t rows, int64_t cols, int transpose,
                hipStream_t stream) {
  g_error.clear();
  if (rows < 1 || cols < 1) return fail(MUON_EINVAL, "rows = %lld, cols = %lld: both must be >= 1", (long long)rows, (long long)cols);
  if (rows > ((int64_t)1 << 40) / cols) return fail(MUON_EINVAL, "rows * cols above 2^40");
  if (transpose != 0 && transpose != 1) return fail(MUON_EINVAL, "transpose = %d is neither 0 nor 1", transpose);
  const char* sn[3] = {"param", "exp_avg", "exp_avg_sq"};
  const char* dn[3] = {"new_param", "new_exp_avg", "new_exp_avg_sq"};
  const size_t b = (size_t)rows * cols * sizeof(float);
  std::vector<Range> r;
  for (int k = 0; k < 3; ++k) {
    if (!src[k] || !dst[k]) return fail(MUON_EINVAL, "%s or %s is NULL", sn[k], dn[k]);
    if ((uintptr_t)src[k] % 4 || (uintptr_t)dst[k] % 4) return fail(MUON_EINVAL, "%s or %s is not 4-byte aligned", sn[k], dn[k]);
    r.push_back({(uintptr_t)dst[k], (uintptr_t)dst[k] + b, 0, dn[k]});
  }
  int rc = check_ranges(r);
  if (rc) return rc;
  // sources may share memory with one another (read only), never with a destination
  for (int k = 0; k < 3; ++k)
    for (int j = 0; j < 3; ++j)
      if ((uintptr_t)src[k] < (uintptr_t)dst[j] + b && (uintptr_t)dst[j] < (uintptr_t)src[k] + b)
        return fail(MUON_EINVAL, "%s overlaps %s", sn[k], dn[j]);
  hipError_t e;
  if (!transpose) {
    for (int k = 0; k < 3; ++k)
      if ((e = hipMemcpyAsync(dst[k], src[k], b, hipMemcpyDeviceToDevice, stream)) != hipSuccess)
        return fail_hip(e, "hipMemcpyAsync(untie)");
    return MUON_OK;
  }
  UntieArgs a{};
  for (int k = 0; k < 3; ++k) {
    a.src[k] = src[k];
    a.dst[k] = dst[k];
  }
  if ((e = launch_untie_transpose(a, rows, cols, stream)) != hipSuccess) return fail_hip(e, "untie kernel launch");
  return MUON_OK;
}

}  // namespace

extern "C" {

int muon_adamw_untie(const float* param, const float* exp_avg, const float* exp_avg_sq, float* new_param,
                     float* new_exp_avg, float* new_exp_avg_sq, int64_t rows, int64_t cols, int transpose,
                     hipStream_t stream) {
  const float* src[3] = {param, exp_avg, exp_avg_sq};
  float* dst[3] = {new_param, new_exp_avg, new_exp_avg_sq};
  return untie_entry(src, dst, rows, cols, transpose, stream);
}

int muon_adamw_step(float* const* params, const float* const* grads, float* const* exp_avg,
                    float* const* exp_avg_sq, const int64_t* numels, const float* weight_decay, int n,
                    float lr, float beta1, float beta2, float eps, int64_t step, hipStream_t stream) {
  return adamw_entry(params, grads, exp_avg, exp_avg_sq, numels, weight_decay, n, lr, beta1, beta2, eps, step,
                     stream);
}

int muon_step_ex(float* const* params, const float* const* grads, float* const* momentum,
                 const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps, const float* coeffs,
                 uint16_t* const* updates, hipStream_t stream) {
  return step_entry(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, 0, updates, stream);
}

int muon_step(float* const* params, const float* const* grads, float* const* momentum,
              const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps, const float* coeffs,
              hipStream_t stream) {
  return step_entry(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, 0, nullptr, stream);
}

int muon_step_sched(float* const* params, const float* const* grads, float* const* momentum,
                    const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps, const float* coeffs,
                    uint16_t* const* updates, hipStream_t stream) {
  return step_entry(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, 3, updates, stream);
}

int muon_newton_schulz(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n,
                       int ns_steps, const float* coeffs, hipStream_t stream) {
  return ns_entry(x, out, shapes, n, ns_steps, coeffs, 0, stream);
}

int muon_newton_schulz_sched(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n,
                             int ns_steps, const float* coeffs, hipStream_t stream) {
  return ns_entry(x, out, shapes, n, ns_steps, coeffs, 3, stream);
}

const char* muon_last_error(void) { return g_error.c_str(); }

size_t muon_workspace_bytes(const muon_shape_t* shapes, int n) {
  g_error.clear();
  if (check_shapes(shapes, n)) return 0;
  return workspace_bytes_of(shapes, n);
}

int muon_set_workspace(void* dev_ptr, size_t bytes) {
  g_error.clear();
  if ((dev_ptr == nullptr) != (bytes == 0)) return fail(MUON_EINVAL, "dev_ptr and bytes must both be set or both be 0");
  if ((uintptr_t)dev_ptr % kAlign) return fail(MUON_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  if (dev_ptr && bytes < kControlBytes) return fail(MUON_ENOMEM, "workspace of %zu bytes is below the %zu-byte minimum", bytes, kControlBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
  clear_plans(st);
  if (st.ws && st.ws_owned) (void)hipFree(st.ws);
  st.ws = dev_ptr;
  st.ws_bytes = bytes;
  st.ws_owned = false;
  if (!dev_ptr) {
    st.ws = nullptr;
    st.ws_bytes = 0;
  }
  return MUON_OK;
}

void muon_release(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_dev) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    kv.second.plans.clear();
    kv.second.adam_plans.clear();
    if (kv.second.ws && kv.second.ws_owned) (void)hipFree(kv.second.ws);
  }
  (void)hipSetDevice(cur);
  g_dev.clear();
  for (hipEvent_t ev : g_ev) (void)hipEventDestroy(ev);
  g_ev.clear();
  g_ev_used = 0;
}

int muon_timing_enable(int kernel) {
  g_error.clear();
  if (kernel < -1 || kernel > MUON_KERNEL_ADAMW) return fail(MUON_EINVAL, "unknown kernel family %d", kernel);
  std::lock_guard<std::mutex> lock(g_mu);
  g_time_kind = kernel;
  g_ev_used = 0;
  return MUON_OK;
}

int muon_timing_read(double* total_ms, int64_t* launches) {
  g_error.clear();
  if (!total_ms || !launches) return fail(MUON_EINVAL, "output pointers must not be NULL");
  std::lock_guard<std::mutex> lock(g_mu);
  double sum = 0.0;
  for (size_t k = 0; k + 1 < g_ev_used; k += 2) {
    hipError_t e = hipEventSynchronize(g_ev[k + 1]);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
    float ms = 0.0f;
    if ((e = hipEventElapsedTime(&ms, g_ev[k], g_ev[k + 1])) != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)(g_ev_used / 2);
  g_ev_used = 0;
  return MUON_OK;
}

}  // extern "C"
