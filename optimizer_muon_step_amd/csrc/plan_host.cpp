// Host plan code: validation, canonical geometry, workspace layout, table
// images and the plan cache.  No GPU calls: device work goes through
// DeviceOps.  The operation itself is described in include/muon.h.
#include "plan_host.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace muon {

namespace {
thread_local std::string g_error;
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

const char* last_error_text() { return g_error.c_str(); }
void clear_error() { g_error.clear(); }

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

namespace {

struct Range {
  uintptr_t lo, hi;
  int mat;
  const char* what;
};

// Every listed array must be disjoint from the others.
int check_ranges(std::vector<Range>& v) {
  std::sort(v.begin(), v.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t k = 1; k < v.size(); ++k)
    if (v[k].lo < v[k - 1].hi)
      return fail(MUON_EINVAL, "%s of matrix %d overlaps %s of matrix %d", v[k].what, v[k].mat, v[k - 1].what,
                  v[k - 1].mat);
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
int64_t gram_tiles(const Geometry& g, int bm) {
  const int64_t t = g.m_pad / bm;
  return t * (t + 1) / 2;
}
int64_t gram_chunks(int64_t slices, int64_t chunk) { return (chunk && slices > chunk) ? (slices + chunk - 1) / chunk : 1; }

// Update tiles of UPD_BM x UPD_BN (the last row tile may hang over m_pad).
int64_t large_update_tiles(const Geometry& g) {
  const int64_t row_units = g.m_pad / UPD_ROWU, step = UPD_BM / UPD_ROWU;
  return (row_units + step - 1) / step * (g.n_pad / UPD_BN);
}

}  // namespace

bool small_call(const muon_shape_t* shapes, int n) {
  int64_t tiles = 0, longest = 0;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    tiles += large_update_tiles(g);
    longest = std::max(longest, gram_slices(g));
  }
  return n > 0 && tiles <= SMALL_MAX_UPD_TILES && longest <= SMALL_MAX_GRAM_SLICES;
}

TileChoice tile_choice(const muon_shape_t* shapes, int n) {
  TileChoice c;
  if (small_call(shapes, n)) {
    c.gram = c.poly = c.upd = TILE_SMALL;
    c.gram_bm = SMALL_SYM;
    return c;
  }
  int64_t gram = 0, poly = 0, upd = 0, upd_med = 0;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    gram += gram_tiles(g, GRAM_BM);
    const int64_t t = g.m_pad / SYM_BM;
    poly += t * (t + 1) / 2;
    upd += large_update_tiles(g);
    upd_med += (int64_t)(g.m_pad / MED_UPD_BM) * (g.n_pad / MED_UPD_BN);
  }
  if (gram < NS_CUS) {
    c.gram = TILE_MEDIUM;
    c.gram_bm = MED_GRAM_BM;
  }
  if (poly <= MED_POLY_MAX_TILES) c.poly = TILE_MEDIUM;
  // A 128 x 256 tile takes about three quarters of a 192 x 256 tile's time
  // (measured 0.73-0.77), so the medium tiles win unless their extra rounds
  // over the CUs cost more than that saves.
  if (3 * ((upd_med + NS_CUS - 1) / NS_CUS) < 4 * ((upd + NS_CUS - 1) / NS_CUS))
    c.upd = upd_med < MED_UPD_MIN_TILES ? TILE_SHALLOW : TILE_MEDIUM;
  return c;
}

namespace {

GramSplit gram_split_of(const muon_shape_t* shapes, int n) {
  GramSplit sp;
  const TileChoice tc = tile_choice(shapes, n);
  if (tc.gram == TILE_SMALL) return sp;
  int64_t total = 0, longest = 0;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    total += gram_tiles(g, tc.gram_bm) * gram_slices(g);
    longest = std::max(longest, gram_slices(g));
  }
  const int64_t share = std::max<int64_t>(GRAM_SPLIT_MIN, (total + NS_CUS - 1) / NS_CUS);
  if (longest <= 2 * share) return sp;
  sp.chunk = share;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    const int64_t nc = gram_chunks(gram_slices(g), sp.chunk);
    if (nc > 1) sp.slots += gram_tiles(g, tc.gram_bm) * nc;
  }
  return sp;
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

}  // namespace

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

int validate_ns(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n, int ns_steps,
                const float* coeffs, int stride) {
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
  return check_ranges(r);
}

int validate_adamw(float* const* params, const float* const* grads, float* const* u, float* const* v,
                   const int64_t* numels, const float* wd, int n, float lr, float beta1, float beta2, float eps,
                   int64_t step) {
  if (n < 0 || n > MUON_ADAMW_MAX_TENSORS) return fail(MUON_EINVAL, "n = %d outside [0, %d]", n, MUON_ADAMW_MAX_TENSORS);
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

int validate_untie(const float* const src[3], float* const dst[3], int64_t rows, int64_t cols, int transpose) {
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
  const int rc = check_ranges(r);
  if (rc) return rc;
  // sources may share memory with one another (read only), never with a destination
  for (int k = 0; k < 3; ++k)
    for (int j = 0; j < 3; ++j)
      if ((uintptr_t)src[k] < (uintptr_t)dst[j] + b && (uintptr_t)dst[j] < (uintptr_t)src[k] + b)
        return fail(MUON_EINVAL, "%s overlaps %s", sn[k], dn[j]);
  return MUON_OK;
}

size_t workspace_bytes_of(const muon_shape_t* shapes, int n) {
  size_t total = kControlBytes;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    total += 2 * g.x_bytes + 2 * g.a_bytes + g.part_bytes;
  }
  const int bm = tile_choice(shapes, n).gram_bm;
  total += align_up((size_t)gram_split_of(shapes, n).slots * bm * bm * sizeof(float));
  return total;
}

std::vector<int> lane_of_matrices(const muon_shape_t* shapes, int n, int max_lanes) {
  std::vector<int> lane(n, 0);
  if (max_lanes <= 1 || n <= 1) return lane;
  // shape groups and their Newton-Schulz cost (m^2 n terms)
  std::vector<std::pair<int64_t, int64_t>> key(n);
  std::vector<std::pair<std::pair<int64_t, int64_t>, double>> groups;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    key[i] = {g.m, g.n};
    const double cost = (double)g.m * g.m * (3.0 * g.n + g.m);
    size_t k = 0;
    while (k < groups.size() && groups[k].first != key[i]) ++k;
    if (k == groups.size()) groups.push_back({key[i], 0.0});
    groups[k].second += cost;
  }
  const int lanes = std::min<int>(std::min(max_lanes, kMaxLanes), (int)groups.size());
  std::stable_sort(groups.begin(), groups.end(), [](const auto& a, const auto& b) { return a.second > b.second; });
  std::vector<double> load(lanes, 0.0);
  std::vector<int> group_lane(groups.size());
  for (size_t k = 0; k < groups.size(); ++k) {
    const int l = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    group_lane[k] = l;
    load[l] += groups[k].second;
  }
  for (int i = 0; i < n; ++i)
    for (size_t k = 0; k < groups.size(); ++k)
      if (groups[k].first == key[i]) lane[i] = group_lane[k];
  return lane;
}

int build_tables(int mode, const muon_shape_t* shapes, int n, char* ws_base, int max_lanes, PlanTables* out) {
  PlanTables& T = *out;
  const std::vector<int> lane_of = lane_of_matrices(shapes, n, max_lanes);
  const int L = n ? *std::max_element(lane_of.begin(), lane_of.end()) + 1 : 1;
  struct Lists {
    std::vector<int32_t> mats, fin;
    std::vector<EwItem> mom, cast, apply;
    std::vector<GemmItem> gram_seq, poly_seq, upd_seq;
    std::vector<int64_t> gram_cost, upd_cost;
    std::vector<RedItem> red;
  };
  std::vector<Lists> lists(L);
  std::vector<MatDesc> desc(n);
  char* cur = ws_base;
  float* scales = reinterpret_cast<float*>(cur);
  cur += kControlBytes;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(shapes[i]);
    MatDesc& d = desc[i];
    Lists& li = lists[lane_of[i]];
    memset(&d, 0, sizeof d);
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
    li.mats.push_back(i);
    if (mode == MODE_STEP) {
      for (int c = 0; c < g.part_cnt; ++c) li.mom.push_back({i, c});
      if (g.part_cnt > NORM_FOLD_MAX) li.fin.push_back(i);
    }
    const int ct = (g.m_pad / CAST_TILE) * (g.n_pad / CAST_TILE);
    for (int t = 0; t < ct; ++t) li.cast.push_back({i, t});
    const int at = g.transposed ? ((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE)
                                : ((g.rows + CAST_WIDE_ROWS - 1) / CAST_WIDE_ROWS) * ((g.cols + CAST_WIDE_COLS - 1) / CAST_WIDE_COLS);
    for (int t = 0; t < at; ++t) li.apply.push_back({i, t});
  }
  // The cast re-reads what the momentum pass just streamed: walking it
  // backwards starts with the lines most likely still in the memory-side
  // cache.
  for (Lists& li : lists) std::reverse(li.cast.begin(), li.cast.end());
  // Partial tiles of split Gram tiles follow the matrices' buffers; the
  // split is decided over the whole call.
  const GramSplit split = gram_split_of(shapes, n);
  const TileChoice tc = tile_choice(shapes, n);
  T.gram_part_off = (size_t)(cur - ws_base);
  (void)carve<float>(cur, (size_t)split.slots * tc.gram_bm * tc.gram_bm);
  // GEMM tiles.  Per matrix in an order that reuses operands (update: all row
  // tiles of one column block in a row, sharing that block of X; symmetric
  // phases: upper-triangle tiles row by row), then spread over the XCDs.
  // Each kind's tile shape comes from tile_choice; a long-K Gram tile may be
  // cut into K chunks, each its own item, summed by the reduce pass.
  T.small = tc.gram == TILE_SMALL;
  T.fused = T.small;
  for (int i = 0; i < n; ++i) T.fused = T.fused && desc[i].m_pad == FUSED_M_PAD;
  T.gram_tile = tc.gram;
  T.poly_tile = tc.poly;
  T.upd_tile = tc.upd;
  T.gram_bm = tc.gram_bm;
  const int gram_bm = tc.gram_bm;
  const int poly_bm = tc.poly == TILE_SMALL ? SMALL_SYM : tc.poly == TILE_MEDIUM ? MED_POLY_BM : SYM_BM;
  const bool upd_small = tc.upd == TILE_SMALL || tc.upd == TILE_SHALLOW;  // both on the small tiles
  const int upd_bm = upd_small ? SMALL_UPD_BM : tc.upd == TILE_MEDIUM ? MED_UPD_BM : UPD_BM;
  const int upd_bn = upd_small ? SMALL_UPD_BN : tc.upd == TILE_MEDIUM ? MED_UPD_BN : UPD_BN;
  int32_t slot = 0;
  for (int i = 0; i < n; ++i) {
    Lists& li = lists[lane_of[i]];
    const int tg = desc[i].m_pad / gram_bm, tm = desc[i].m_pad / poly_bm, tn = desc[i].n_pad / upd_bn;
    const int64_t ks = ((int64_t)desc[i].n + 63) / 64;                   // Gram K slices
    const int32_t kp = (int32_t)(((int64_t)desc[i].m + SYM_BK - 1) / SYM_BK);  // poly K slices
    const int32_t ku = (int32_t)(2 * (((int64_t)desc[i].m + 127) / 128));  // update: even, see the kernel
    const int64_t nc = gram_chunks(ks, split.chunk);
    for (int ti = 0; ti < tg; ++ti)
      for (int tj = ti; tj < tg; ++tj) {
        if (nc == 1) {
          li.gram_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, (int32_t)ks, -1});
          li.gram_cost.push_back(ks);
          continue;
        }
        for (int64_t c = 0; c < nc; ++c) {
          const int64_t a = ks * c / nc, b = ks * (c + 1) / nc;
          li.gram_seq.push_back({i, (int16_t)ti, (int16_t)tj, (int32_t)a, (int32_t)(b - a), slot + (int32_t)c});
          li.gram_cost.push_back(b - a);
        }
        const int SUB = gram_bm / RED_TILE;
        for (int bi = 0; bi < SUB; ++bi)
          for (int bj = 0; bj < SUB; ++bj)
            if (ti != tj || bi <= bj)
              li.red.push_back({i, (int16_t)ti, (int16_t)tj, slot, (int16_t)nc, (int8_t)bi, (int8_t)bj});
        slot += (int32_t)nc;
      }
    for (int ti = 0; ti < tm; ++ti)
      for (int tj = ti; tj < tm; ++tj) li.poly_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, kp, -1});
    for (int tj = 0; tj < tn; ++tj)
      for (int ti = 0; ti < desc[i].m_pad / UPD_ROWU; ti += upd_bm / UPD_ROWU) {
        li.upd_seq.push_back({i, (int16_t)ti, (int16_t)tj, 0, ku, -1});
        li.upd_cost.push_back(ku);
      }
  }
  if (slot != split.slots)
    return fail(MUON_EINVAL, "internal: %d Gram partial tiles planned, %lld sized", slot, (long long)split.slots);

  size_t off = 0;
  auto place = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  T.o_desc = place(sizeof(MatDesc) * n);
  T.n_mat = n;
  T.lanes.assign(L, LaneTables{});
  std::vector<std::vector<GemmItem>> gram(L), poly(L), upd(L);
  size_t items = 0;
  for (int l = 0; l < L; ++l) {
    Lists& li = lists[l];
    std::vector<int64_t> poly_cost(li.poly_seq.size());
    for (size_t k = 0; k < li.poly_seq.size(); ++k) poly_cost[k] = li.poly_seq[k].kn;
    gram[l] = xcd_interleave(li.gram_seq, li.gram_cost);
    poly[l] = xcd_interleave(li.poly_seq, poly_cost);
    upd[l] = xcd_interleave(li.upd_seq, li.upd_cost);
    LaneTables& lt = T.lanes[l];
    lt.o_mats = place(sizeof(int32_t) * li.mats.size());
    lt.o_fin = place(sizeof(int32_t) * li.fin.size());
    lt.o_mom = place(sizeof(EwItem) * li.mom.size());
    lt.o_cast = place(sizeof(EwItem) * li.cast.size());
    lt.o_apply = place(sizeof(EwItem) * li.apply.size());
    lt.o_gram = place(sizeof(GemmItem) * gram[l].size());
    lt.o_poly = place(sizeof(GemmItem) * poly[l].size());
    lt.o_upd = place(sizeof(GemmItem) * upd[l].size());
    lt.o_red = place(sizeof(RedItem) * li.red.size());
    lt.n_mats = (int)li.mats.size();
    lt.n_fin = (int)li.fin.size();
    lt.n_mom = (int)li.mom.size();
    lt.n_cast = (int)li.cast.size();
    lt.n_apply = (int)li.apply.size();
    lt.n_gram = (int)gram[l].size();
    lt.n_poly = (int)poly[l].size();
    lt.n_upd = (int)upd[l].size();
    lt.n_red = (int)li.red.size();
    items += li.mom.size() + li.cast.size() + li.apply.size() + gram[l].size() + poly[l].size() + upd[l].size() +
             li.red.size();
  }
  if (items > (size_t)INT32_MAX / 2) return fail(MUON_EINVAL, "call of %zu work items is too large", items);
  T.image.assign(std::max<size_t>(off, kAlign), 0);
  char* h = T.image.data();
  auto put = [&](size_t o, const void* src, size_t bytes) {
    if (bytes) memcpy(h + o, src, bytes);
  };
  put(T.o_desc, desc.data(), sizeof(MatDesc) * n);
  for (int l = 0; l < L; ++l) {
    const Lists& li = lists[l];
    const LaneTables& lt = T.lanes[l];
    put(lt.o_mats, li.mats.data(), sizeof(int32_t) * li.mats.size());
    put(lt.o_fin, li.fin.data(), sizeof(int32_t) * li.fin.size());
    put(lt.o_mom, li.mom.data(), sizeof(EwItem) * li.mom.size());
    put(lt.o_cast, li.cast.data(), sizeof(EwItem) * li.cast.size());
    put(lt.o_apply, li.apply.data(), sizeof(EwItem) * li.apply.size());
    put(lt.o_gram, gram[l].data(), sizeof(GemmItem) * gram[l].size());
    put(lt.o_poly, poly[l].data(), sizeof(GemmItem) * poly[l].size());
    put(lt.o_upd, upd[l].data(), sizeof(GemmItem) * upd[l].size());
    put(lt.o_red, li.red.data(), sizeof(RedItem) * li.red.size());
  }
  return MUON_OK;
}

void make_ptr_records(int mode, const muon_shape_t* shapes, int n, float* const* params, const float* const* grads,
                      float* const* moms, uint16_t* const* upd, const uint16_t* const* xin,
                      std::vector<PtrRecord>* out) {
  out->assign(n, PtrRecord{});
  for (int i = 0; i < n; ++i) {
    PtrRecord& r = (*out)[i];
    r.mat = i;
    r.W = params ? params[i] : nullptr;
    r.G = grads ? grads[i] : nullptr;
    r.M = moms ? moms[i] : nullptr;
    r.upd = upd ? upd[i] : nullptr;
    r.xin = xin ? xin[i] : nullptr;
    const bool cols4 = shapes[i].cols % 4 == 0;
    if (mode == MODE_STEP)
      r.vec4 = cols4 && (uintptr_t)r.W % 16 == 0 && (uintptr_t)r.G % 16 == 0 && (uintptr_t)r.M % 16 == 0;
    else
      r.vec4 = cols4 && (uintptr_t)r.xin % 8 == 0;
  }
}

bool same_records(const std::vector<PtrRecord>& a, const std::vector<PtrRecord>& b) {
  if (a.size() != b.size()) return false;
  for (size_t i = 0; i < a.size(); ++i)
    if (a[i].W != b[i].W || a[i].G != b[i].G || a[i].M != b[i].M || a[i].upd != b[i].upd || a[i].xin != b[i].xin ||
        a[i].vec4 != b[i].vec4 || a[i].mat != b[i].mat)
      return false;
  return true;
}

// ---------------------------------------------------------------- cache ----

PlanCache::~PlanCache() { release_all(); }

void PlanCache::free_plan(Plan* p) {
  if (p->dev || p->host) ops_->free_tables(p->dev, p->host);
  p->dev = p->host = nullptr;
}

void PlanCache::release_all() {
  for (auto& p : plans_) free_plan(p.get());
  plans_.clear();
  for (void* w : retired_) ops_->free_workspace(w);
  retired_.clear();
  if (ws_ && ws_owned_) ops_->free_workspace(ws_);
  ws_ = nullptr;
  ws_bytes_ = 0;
  ws_owned_ = false;
}

// Free every uncaptured plan on workspace ws (the device is idle).
void PlanCache::drop_uncaptured_on(char* ws) {
  for (auto it = plans_.begin(); it != plans_.end();) {
    if ((*it)->ws == ws && !(*it)->captured) {
      free_plan(it->get());
      it = plans_.erase(it);
    } else {
      ++it;
    }
  }
}

int PlanCache::acquire_workspace(size_t need, bool capturing) {
  if (ws_ && ws_bytes_ >= need) return MUON_OK;
  if (ws_ && !ws_owned_)
    return fail(MUON_ENOMEM, "caller workspace has %zu bytes, this call needs %zu", ws_bytes_, need);
  if (capturing)
    return fail(MUON_EINVAL, "this call needs a %zu-byte workspace (%zu now): make one call with these shapes "
                "before capturing it into a graph", need, ws_bytes_);
  if (ws_) {
    // Growing: wait for work that may still use the old buffer.  Plans that
    // a captured graph uses keep it (retired, freed at release).
    int rc = ops_->sync_device();
    ++stats.syncs;
    if (rc) return rc;
    drop_uncaptured_on(ws_);
    bool held = false;
    for (auto& p : plans_) held = held || p->ws == ws_;
    if (held)
      retired_.push_back(ws_);
    else
      ops_->free_workspace(ws_);
    ws_ = nullptr;
    ws_bytes_ = 0;
  }
  void* p = nullptr;
  const int rc = ops_->alloc_workspace(need, &p);
  if (rc) return rc;
  ++stats.ws_allocs;
  ws_ = static_cast<char*>(p);
  ws_bytes_ = need;
  ws_owned_ = true;
  return MUON_OK;
}

int PlanCache::set_workspace(void* p, size_t bytes) {
  const int rc = ops_->sync_device();
  ++stats.syncs;
  if (rc) return rc;
  if (ws_) {
    drop_uncaptured_on(ws_);
    bool held = false;
    for (auto& q : plans_) held = held || q->ws == ws_;
    if (ws_owned_) {
      if (held)
        retired_.push_back(ws_);
      else
        ops_->free_workspace(ws_);
    }
  }
  ws_ = static_cast<char*>(p);
  ws_bytes_ = p ? bytes : 0;
  ws_owned_ = false;
  return MUON_OK;
}

int PlanCache::prepare(int mode, const muon_shape_t* shapes, int n, int max_lanes, const std::vector<PtrRecord>& recs,
                       bool capturing, Plan** out) {
  int rc = acquire_workspace(workspace_bytes_of(shapes, n), capturing);
  if (rc) return rc;
  std::vector<int64_t> key;
  key.reserve(4 + 2 * (size_t)n);
  key.push_back(mode);
  key.push_back(max_lanes);
  key.push_back(n);
  key.push_back((int64_t)(uintptr_t)ws_);
  for (int i = 0; i < n; ++i) {
    key.push_back(shapes[i].rows);
    key.push_back(shapes[i].cols);
  }
  Plan* plan = nullptr;
  for (auto it = plans_.begin(); it != plans_.end(); ++it) {
    if ((*it)->key == key) {
      if (it != plans_.begin()) plans_.splice(plans_.begin(), plans_, it);
      plan = plans_.front().get();
      break;
    }
  }
  if (!plan) {
    if (capturing)
      return fail(MUON_EINVAL, "no plan for these shapes yet: make one call with them before capturing it into a graph");
    auto p = std::make_unique<Plan>();
    p->key = std::move(key);
    p->ws = ws_;
    if ((rc = build_tables(mode, shapes, n, ws_, max_lanes, &p->t))) return rc;
    if ((rc = ops_->alloc_tables(p->t.image.size(), &p->dev, &p->host))) return rc;
    if ((rc = ops_->upload(p->dev, p->host, p->t.image.data(), p->t.image.size()))) {
      free_plan(p.get());
      return rc;
    }
    ++stats.plan_builds;
    ++stats.uploads;
    plans_.push_front(std::move(p));
    plan = plans_.front().get();
    // Keep at most kMaxPlans uncaptured plans; the least recently used goes
    // once the device is done with it.
    size_t uncaptured = 0;
    for (auto& q : plans_) uncaptured += q->captured ? 0 : 1;
    if (uncaptured > kMaxPlans) {
      for (auto it = std::prev(plans_.end());; --it) {
        if (!(*it)->captured && it->get() != plan) {
          rc = ops_->sync_device();
          ++stats.syncs;
          if (rc) return rc;
          free_plan(it->get());
          plans_.erase(it);
          ++stats.evictions;
          break;
        }
        if (it == plans_.begin()) break;
      }
    }
  }
  if (capturing) plan->captured = true;
  // Patch the caller pointers unless the descriptors already hold exactly
  // these (known only for plans no graph writes into).
  if (capturing || plan->captured || !plan->ptrs_known || !same_records(plan->ptrs, recs)) {
    if (!capturing) plan->ptrs_known = false;
    for (int i = 0; i < n; i += PATCH_MAX) {
      const int cnt = std::min(PATCH_MAX, n - i);
      if ((rc = ops_->patch(plan->at<char>(plan->t.o_desc), recs.data() + i, cnt))) return rc;
      ++stats.patch_calls;
    }
    if (!capturing) {
      plan->ptrs = recs;
      plan->ptrs_known = true;
    }
  }
  *out = plan;
  return MUON_OK;
}

}  // namespace muon
