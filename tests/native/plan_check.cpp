// Host check of the plan code (csrc/plan_host.cpp) against a fake device
// whose memory is ordinary host memory: built with the host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_plan_host.py.
// Every table the cache uploads and every pointer patch it issues is applied
// to that memory, so out-of-bounds table writes, leaks and undefined
// behaviour in the plan code show up here.  Prints "ok" and exits 0 when
// every check holds.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "plan_host.h"

using namespace muon;

static int g_failures = 0;
#define CHECK(cond)                                                                   \
  do {                                                                                \
    if (!(cond)) {                                                                    \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                                   \
    }                                                                                 \
  } while (0)

// Device memory is host memory; stream-ordered operations apply at once.
class FakeOps : public DeviceOps {
 public:
  std::map<void*, size_t> live;  // device and host blocks still allocated
  int64_t syncs = 0, uploads = 0, patches = 0;
  bool fail_alloc = false;

  void* grab(size_t bytes) {
    void* p = std::malloc(bytes);
    std::memset(p, 0xCD, bytes);  // like device memory: not zeroed
    live[p] = bytes;
    return p;
  }
  void drop(void* p) {
    if (!p) return;
    CHECK(live.count(p) == 1);
    live.erase(p);
    std::free(p);
  }
  int alloc_tables(size_t bytes, void** dev, void** host) override {
    if (fail_alloc) return fail(MUON_ENOMEM, "fake allocation failure");
    *dev = grab(bytes);
    *host = grab(bytes);
    return MUON_OK;
  }
  void free_tables(void* dev, void* host) override {
    drop(dev);
    drop(host);
  }
  int upload(void* dev, void* host, const void* image, size_t bytes) override {
    CHECK(live.count(dev) && live[dev] >= bytes && live.count(host) && live[host] >= bytes);
    std::memcpy(host, image, bytes);
    std::memcpy(dev, host, bytes);
    ++uploads;
    return MUON_OK;
  }
  int patch(void* dev_desc, const PtrRecord* recs, int count) override {
    CHECK(count >= 1 && count <= PATCH_MAX);
    MatDesc* d = static_cast<MatDesc*>(dev_desc);
    for (int k = 0; k < count; ++k) {
      MatDesc& m = d[recs[k].mat];
      m.W = recs[k].W;
      m.G = recs[k].G;
      m.M = recs[k].M;
      m.upd = recs[k].upd;
      m.xin = recs[k].xin;
      m.vec4 = recs[k].vec4;
    }
    ++patches;
    return MUON_OK;
  }
  int alloc_workspace(size_t bytes, void** p) override {
    if (fail_alloc) return fail(MUON_ENOMEM, "fake allocation failure");
    *p = grab(bytes);
    return MUON_OK;
  }
  void free_workspace(void* p) override { drop(p); }
  int sync_device() override {
    ++syncs;
    return MUON_OK;
  }
};

static std::vector<muon_shape_t> shapes_of(std::initializer_list<std::pair<int64_t, int64_t>> l) {
  std::vector<muon_shape_t> v;
  for (auto& p : l) v.push_back({p.first, p.second});
  return v;
}

static std::vector<muon_shape_t> gpt2_block(int layers) {
  std::vector<muon_shape_t> v;
  for (int l = 0; l < layers; ++l) {
    v.push_back({768, 2304});
    v.push_back({768, 768});
    v.push_back({768, 3072});
    v.push_back({3072, 768});
  }
  return v;
}

// Fake caller pointers: distinct, 256-byte aligned, never dereferenced.
static std::vector<PtrRecord> records(const std::vector<muon_shape_t>& s, uintptr_t base) {
  std::vector<float*> W, M;
  std::vector<const float*> G;
  for (size_t i = 0; i < s.size(); ++i) {
    W.push_back(reinterpret_cast<float*>(base + 0x1000000 * (3 * i + 1)));
    G.push_back(reinterpret_cast<const float*>(base + 0x1000000 * (3 * i + 2)));
    M.push_back(reinterpret_cast<float*>(base + 0x1000000 * (3 * i + 3)));
  }
  std::vector<PtrRecord> r;
  make_ptr_records(MODE_STEP, s.data(), (int)s.size(), W.data(), G.data(), M.data(), nullptr, nullptr, &r);
  return r;
}

// Every table of a plan is consistent with the shapes and stays inside the
// workspace and the table block.
static void check_tables(const Plan& p, const std::vector<muon_shape_t>& s, size_t ws_bytes) {
  const PlanTables& t = p.t;
  const int n = (int)s.size();
  CHECK(t.n_mat == n);
  CHECK(t.image.size() % 256 == 0);
  const MatDesc* d = p.at<MatDesc>(t.o_desc);
  const char* ws_lo = p.ws;
  const char* ws_hi = p.ws + ws_bytes;
  std::vector<std::pair<const char*, const char*>> regions;
  int64_t mom = 0, cast = 0, apply = 0;
  for (int i = 0; i < n; ++i) {
    const Geometry g = geometry_of(s[i]);
    CHECK(d[i].rows == s[i].rows && d[i].cols == s[i].cols);
    CHECK(d[i].m <= d[i].n && d[i].m_pad % NS_PAD_M == 0 && d[i].n_pad % NS_PAD_N == 0);
    CHECK(d[i].transposed == (s[i].rows > s[i].cols));
    const char* r[5][2] = {{(const char*)d[i].X[0], (const char*)d[i].X[0] + g.x_bytes},
                           {(const char*)d[i].X[1], (const char*)d[i].X[1] + g.x_bytes},
                           {(const char*)d[i].A, (const char*)d[i].A + g.a_bytes},
                           {(const char*)d[i].B, (const char*)d[i].B + g.a_bytes},
                           {(const char*)d[i].part, (const char*)d[i].part + g.part_bytes}};
    for (auto& q : r) {
      CHECK(q[0] >= ws_lo + kControlBytes && q[1] <= ws_hi);
      CHECK((uintptr_t)q[0] % 256 == 0);
      regions.push_back({q[0], q[1]});
    }
    CHECK((const char*)d[i].scale >= ws_lo && (const char*)(d[i].scale + 1) <= ws_lo + kControlBytes);
    mom += g.part_cnt;
    cast += (int64_t)(g.m_pad / CAST_TILE) * (g.n_pad / CAST_TILE);
    apply += g.transposed ? (int64_t)((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE)
                          : (int64_t)((g.rows + CAST_WIDE_ROWS - 1) / CAST_WIDE_ROWS) *
                                ((g.cols + CAST_WIDE_COLS - 1) / CAST_WIDE_COLS);
  }
  std::sort(regions.begin(), regions.end());
  for (size_t k = 1; k < regions.size(); ++k) CHECK(regions[k].first >= regions[k - 1].second);
  // every matrix in exactly one lane's list; lanes hold whole shape groups
  std::vector<int> lane_of(n, -1);
  int64_t n_mom = 0, n_cast = 0, n_apply = 0;
  for (size_t l = 0; l < t.lanes.size(); ++l) {
    const LaneTables& lt = t.lanes[l];
    const int32_t* mats = p.at<int32_t>(lt.o_mats);
    CHECK(lt.n_mats >= 1);
    for (int k = 0; k < lt.n_mats; ++k) {
      CHECK(mats[k] >= 0 && mats[k] < n);
      if (mats[k] < 0 || mats[k] >= n) continue;
      CHECK(lane_of[mats[k]] == -1);
      lane_of[mats[k]] = (int)l;
    }
    n_mom += lt.n_mom;
    n_cast += lt.n_cast;
    n_apply += lt.n_apply;
  }
  // the finalisation list: in the step mode exactly the matrices with more
  // than NORM_FOLD_MAX norm partials, each once, in its own lane
  std::vector<int> fin_seen(n, 0);
  for (size_t l = 0; l < t.lanes.size(); ++l) {
    const LaneTables& lt = t.lanes[l];
    const int32_t* fin = p.at<int32_t>(lt.o_fin);
    for (int k = 0; k < lt.n_fin; ++k) {
      CHECK(fin[k] >= 0 && fin[k] < n);
      if (fin[k] < 0 || fin[k] >= n) continue;
      CHECK(lane_of[fin[k]] == (int)l);
      ++fin_seen[fin[k]];
    }
  }
  const bool step_mode = !p.key.empty() && p.key[0] == MODE_STEP;
  for (int i = 0; i < n; ++i)
    CHECK(fin_seen[i] == ((step_mode && geometry_of(s[i]).part_cnt > NORM_FOLD_MAX) ? 1 : 0));
  for (int i = 0; i < n; ++i) {
    CHECK(lane_of[i] >= 0);
    for (int j = 0; j < n; ++j) {
      const Geometry a = geometry_of(s[i]), b = geometry_of(s[j]);
      if (a.m == b.m && a.n == b.n) CHECK(lane_of[i] == lane_of[j]);
    }
  }
  CHECK(n_mom == mom && n_cast == cast && n_apply == apply);
  // elementwise items: each (matrix, index) once over all lanes, in the
  // lane of its matrix, indices in range
  auto ew = [&](size_t off, int cnt, int which, int lane, std::set<std::pair<int, int>>& seen) {
    const EwItem* it = p.at<EwItem>(off);
    for (int k = 0; k < cnt; ++k) {
      CHECK(it[k].mat >= 0 && it[k].mat < n);
      if (it[k].mat < 0 || it[k].mat >= n) continue;
      CHECK(lane_of[it[k].mat] == lane);
      const Geometry g = geometry_of(s[it[k].mat]);
      const int lim = which == 0 ? g.part_cnt
                      : which == 1 ? (g.m_pad / CAST_TILE) * (g.n_pad / CAST_TILE)
                     : g.transposed ? ((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE)
                                    : ((g.rows + CAST_WIDE_ROWS - 1) / CAST_WIDE_ROWS) *
                                          ((g.cols + CAST_WIDE_COLS - 1) / CAST_WIDE_COLS);
      CHECK(it[k].idx >= 0 && it[k].idx < lim);
      CHECK(seen.insert({it[k].mat, it[k].idx}).second);
    }
  };
  std::set<std::pair<int, int>> seen_mom, seen_cast, seen_apply;
  for (size_t l = 0; l < t.lanes.size(); ++l) {
    ew(t.lanes[l].o_mom, t.lanes[l].n_mom, 0, (int)l, seen_mom);
    ew(t.lanes[l].o_cast, t.lanes[l].n_cast, 1, (int)l, seen_cast);
    ew(t.lanes[l].o_apply, t.lanes[l].n_apply, 2, (int)l, seen_apply);
  }
  // GEMM items: tiles inside the padded matrix, K ranges inside the true
  // size, each output tile covered once per kind (Gram chunks tile K)
  CHECK(t.small == small_call(s.data(), n));
  bool fused = t.small;
  for (int i = 0; i < n; ++i) fused = fused && geometry_of(s[i]).m_pad == FUSED_M_PAD;
  CHECK(t.fused == fused);
  // tile kinds: all small in a small call, else each kind large or medium by
  // its own tile count
  {
    int64_t g256 = 0, p128 = 0, u192 = 0, u128 = 0;
    for (int i = 0; i < n; ++i) {
      const Geometry g = geometry_of(s[i]);
      g256 += (int64_t)(g.m_pad / 256) * (g.m_pad / 256 + 1) / 2;
      p128 += (int64_t)(g.m_pad / 128) * (g.m_pad / 128 + 1) / 2;
      u192 += (int64_t)((g.m_pad / 64 + 2) / 3) * (g.n_pad / 256);
      u128 += (int64_t)(g.m_pad / 128) * (g.n_pad / 256);
    }
    if (t.small) {
      CHECK(t.gram_tile == TILE_SMALL && t.poly_tile == TILE_SMALL && t.upd_tile == TILE_SMALL && t.gram_bm == 64);
    } else {
      CHECK(t.gram_tile == (g256 < 256 ? TILE_MEDIUM : TILE_LARGE));
      CHECK(t.gram_bm == (g256 < 256 ? 128 : 256));
      CHECK(t.poly_tile == (p128 <= 128 ? TILE_MEDIUM : TILE_LARGE));
      const bool med = 3 * ((u128 + 255) / 256) < 4 * ((u192 + 255) / 256);
      CHECK(t.upd_tile == (!med ? TILE_LARGE : u128 <= 128 ? TILE_SHALLOW : TILE_MEDIUM));
    }
  }
  const int gram_bm = t.gram_bm;
  const int poly_bm = t.poly_tile == TILE_SMALL ? 64 : t.poly_tile == TILE_MEDIUM ? 64 : 128;
  const bool upd_small = t.upd_tile == TILE_SMALL || t.upd_tile == TILE_SHALLOW;
  const int upd_bm = upd_small ? 64 : t.upd_tile == TILE_MEDIUM ? 128 : 192;
  const int upd_bn = upd_small ? 128 : 256;
  std::map<std::tuple<int, int, int>, int64_t> ksum[3];
  auto gemm = [&](size_t off, int cnt, int kind, int lane) {
    const GemmItem* it = p.at<GemmItem>(off);
    CHECK(cnt % 8 == 0);
    for (int k = 0; k < cnt; ++k) {
      if (it[k].mat < 0) continue;
      CHECK(it[k].mat < n);
      if (it[k].mat >= n) continue;
      CHECK(lane_of[it[k].mat] == lane);
      const MatDesc& m = d[it[k].mat];
      if (kind == 0) {
        CHECK(it[k].ti <= it[k].tj && (it[k].tj + 1) * gram_bm <= m.m_pad);
        CHECK(!t.small || it[k].slot < 0);
        CHECK(it[k].k0 >= 0 && (int64_t)(it[k].k0 + it[k].kn) * 64 <= m.n_pad && it[k].kn >= 1);
        ksum[0][{it[k].mat, it[k].ti, it[k].tj}] += it[k].kn;
        if (it[k].slot >= 0) {
          const char* lo = p.ws + t.gram_part_off + (size_t)it[k].slot * gram_bm * gram_bm * 4;
          CHECK(lo >= p.ws && lo + (size_t)gram_bm * gram_bm * 4 <= ws_hi);
        }
      } else if (kind == 1) {
        CHECK(it[k].ti <= it[k].tj && (it[k].tj + 1) * poly_bm <= m.m_pad && it[k].kn * SYM_BK <= m.m_pad);
        CHECK((int64_t)it[k].kn * SYM_BK >= m.m);
        ksum[1][{it[k].mat, it[k].ti, it[k].tj}] += 1;
      } else {
        CHECK(it[k].ti * UPD_ROWU < m.m_pad && (it[k].tj + 1) * upd_bn <= m.n_pad);
        CHECK(it[k].ti % (upd_bm / UPD_ROWU) == 0);
        CHECK(it[k].kn % 2 == 0 && it[k].kn * 64 <= m.m_pad);
        CHECK(it[k].ti * UPD_ROWU + upd_bm <= m.m_pad + NS_PAD_M);  // overhang inside the spare rows
        ksum[2][{it[k].mat, it[k].ti, it[k].tj}] += 1;
      }
    }
  };
  for (size_t l = 0; l < t.lanes.size(); ++l) {
    gemm(t.lanes[l].o_gram, t.lanes[l].n_gram, 0, (int)l);
    gemm(t.lanes[l].o_poly, t.lanes[l].n_poly, 1, (int)l);
    gemm(t.lanes[l].o_upd, t.lanes[l].n_upd, 2, (int)l);
  }
  for (auto& kv : ksum[0]) CHECK(kv.second == ((int64_t)d[std::get<0>(kv.first)].n + 63) / 64);
  for (int kind = 1; kind < 3; ++kind)
    for (auto& kv : ksum[kind]) CHECK(kv.second == 1);
  int64_t want_poly = 0, want_gram = 0, want_upd = 0;
  for (int i = 0; i < n; ++i) {
    want_poly += (int64_t)(d[i].m_pad / poly_bm) * (d[i].m_pad / poly_bm + 1) / 2;
    want_gram += (int64_t)(d[i].m_pad / gram_bm) * (d[i].m_pad / gram_bm + 1) / 2;
    want_upd += (int64_t)(d[i].m_pad / UPD_ROWU + upd_bm / UPD_ROWU - 1) / (upd_bm / UPD_ROWU) * (d[i].n_pad / upd_bn);
  }
  CHECK((int64_t)ksum[0].size() == want_gram && (int64_t)ksum[1].size() == want_poly &&
        (int64_t)ksum[2].size() == want_upd);
}

static void check_pointers(const Plan& p, const std::vector<PtrRecord>& r) {
  const MatDesc* d = p.at<MatDesc>(p.t.o_desc);
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(d[i].W == r[i].W && d[i].G == r[i].G && d[i].M == r[i].M && d[i].vec4 == r[i].vec4);
  }
}

static void test_validation() {
  const auto good = shapes_of({{4, 4}});
  float* W[1] = {reinterpret_cast<float*>(0x10000)};
  const float* G[1] = {reinterpret_cast<const float*>(0x20000)};
  float* M[1] = {reinterpret_cast<float*>(0x30000)};
  const float c[3] = {3.4445f, -4.775f, 2.0315f};
  CHECK(validate_step(W, G, M, good.data(), 1, 0.02f, 0.95f, 5, c, 0, nullptr) == MUON_OK);
  CHECK(validate_step(nullptr, G, M, good.data(), 1, 0.02f, 0.95f, 5, c, 0, nullptr) == MUON_EINVAL);
  CHECK(validate_step(W, G, M, good.data(), 1, 0.02f, 1.0f, 5, c, 0, nullptr) == MUON_EINVAL);
  CHECK(validate_step(W, G, M, good.data(), 1, 0.02f, 0.95f, 65, c, 0, nullptr) == MUON_EINVAL);
  CHECK(validate_step(W, G, M, good.data(), 1, 0.02f, 0.95f, 2, nullptr, 3, nullptr) == MUON_EINVAL);
  float* M2[1] = {reinterpret_cast<float*>(0x10008)};  // overlaps W
  CHECK(validate_step(W, G, M2, good.data(), 1, 0.02f, 0.95f, 5, c, 0, nullptr) == MUON_EINVAL);
  CHECK(std::string(last_error_text()).find("overlaps") != std::string::npos);
  const auto bad = shapes_of({{1 << 16, 1 << 16}});
  CHECK(check_shapes(bad.data(), 1) == MUON_EINVAL);
  const auto zero = shapes_of({{0, 5}});
  CHECK(check_shapes(zero.data(), 1) == MUON_EINVAL);
  CHECK(check_shapes(nullptr, 1) == MUON_EINVAL);
  CHECK(check_shapes(nullptr, 0) == MUON_OK);
  const float nanc[3] = {1.0f, __builtin_nanf(""), 0.0f};
  CHECK(check_coeffs(nanc, 5, 0) == MUON_EINVAL);
  int64_t numel[1] = {8};
  float wd[1] = {-1.0f};
  CHECK(validate_adamw(W, G, M, M, numel, wd, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 1) == MUON_EINVAL);
  const float* src[3] = {G[0], G[0], G[0]};
  float* dst[3] = {W[0], M[0], reinterpret_cast<float*>(0x40000)};
  CHECK(validate_untie(src, dst, 4, 4, 1) == MUON_OK);
  CHECK(validate_untie(src, dst, 4, 4, 2) == MUON_EINVAL);
}

static void test_tables_of_many_shapes() {
  const std::vector<std::vector<muon_shape_t>> sets = {
      shapes_of({{256, 512}}),
      gpt2_block(1),
      gpt2_block(12),
      shapes_of({{50257, 768}, {768, 768}}),
      shapes_of({{1, 1}, {1, 7}, {7, 1}, {129, 1000}, {300, 200}, {5, 4099}, {257, 129}, {300, 1}}),
      shapes_of({{64, 4100}, {512, 20000}, {20001, 300}}),
  };
  for (const auto& s : sets) {
    FakeOps ops;
    {
      PlanCache cache(&ops);
      const auto r = records(s, 0x7f0000000000ull);
      Plan* p = nullptr;
      CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, r, false, &p) == MUON_OK);
      if (!p) continue;
      check_tables(*p, s, cache.workspace_bytes());
      check_pointers(*p, r);
      CHECK(cache.workspace_bytes() == workspace_bytes_of(s.data(), (int)s.size()));
    }
    CHECK(ops.live.empty());  // the cache freed everything it allocated
  }
}

static void test_pointer_alternation_needs_no_rebuild() {
  FakeOps ops;
  PlanCache cache(&ops);
  const auto s = gpt2_block(12);
  const auto a = records(s, 0x7f0000000000ull), b = records(s, 0x7e0000000000ull);
  Plan* p = nullptr;
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, a, false, &p) == MUON_OK);
  const CacheStats first = cache.stats;
  CHECK(first.plan_builds == 1 && first.uploads == 1 && first.syncs == 0 && first.ws_allocs == 1);
  CHECK(first.patch_calls == 2);  // 48 matrices, 40 per patch
  // the same pointers again: nothing but the launches
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, a, false, &p) == MUON_OK);
  CHECK(cache.stats.patch_calls == first.patch_calls);
  for (int k = 0; k < 10; ++k) {
    const auto& r = (k % 2) ? a : b;
    Plan* q = nullptr;
    CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, r, false, &q) == MUON_OK);
    CHECK(q == p);
    check_pointers(*q, r);
  }
  CHECK(cache.stats.plan_builds == 1 && cache.stats.syncs == 0 && cache.stats.uploads == 1);
  CHECK(cache.stats.patch_calls == first.patch_calls + 10 * 2);
  // the NS-only entry on the same shapes is a plan of its own
  std::vector<PtrRecord> x;
  std::vector<uint16_t*> out(s.size(), reinterpret_cast<uint16_t*>(0x1000));
  std::vector<const uint16_t*> in(s.size(), reinterpret_cast<const uint16_t*>(0x2000));
  make_ptr_records(MODE_NS, s.data(), (int)s.size(), nullptr, nullptr, nullptr, out.data(), in.data(), &x);
  CHECK(cache.prepare(MODE_NS, s.data(), (int)s.size(), 3, x, false, &p) == MUON_OK);
  CHECK(cache.stats.plan_builds == 2 && cache.stats.syncs == 0);
}

static void test_eviction_and_capture() {
  FakeOps ops;
  {
    PlanCache cache(&ops);
    // plan 0 is captured after one eager call
    const auto s0 = shapes_of({{64, 64}});
    const auto r0 = records(s0, 0x7f0000000000ull);
    Plan* p0 = nullptr;
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, 3, r0, true, &p0) == MUON_EINVAL);  // never seen: refused
    CHECK(cache.stats.plan_builds == 0);
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, 3, r0, false, &p0) == MUON_OK);
    const int64_t before = cache.stats.patch_calls;
    Plan* pc = nullptr;
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, 3, r0, true, &pc) == MUON_OK);
    CHECK(pc == p0 && pc->captured);
    CHECK(cache.stats.patch_calls == before + 1);  // a capture always records the pointer write
    // eager calls on a captured plan always re-patch (a replay writes its own pointers)
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, 3, r0, false, &pc) == MUON_OK);
    CHECK(cache.stats.patch_calls == before + 2);
    // a larger set of shapes refused under capture (it would allocate)
    const auto big = gpt2_block(1);
    const auto rb = records(big, 0x7d0000000000ull);
    Plan* pb = nullptr;
    CHECK(cache.prepare(MODE_STEP, big.data(), (int)big.size(), 3, rb, true, &pb) == MUON_EINVAL);
    // ... fine eagerly: the workspace grows, the captured plan keeps the old one
    char* old_ws = p0->ws;
    CHECK(cache.prepare(MODE_STEP, big.data(), (int)big.size(), 3, rb, false, &pb) == MUON_OK);
    CHECK(cache.stats.syncs == 1);
    CHECK(ops.live.count(old_ws) == 1);  // retired, not freed
    CHECK(p0->captured && p0->ws == old_ws);
    // nine more shape sets: uncaptured plans are evicted, the captured one stays
    for (int k = 0; k < 9; ++k) {
      const auto s = shapes_of({{32 + k, 48}});
      const auto r = records(s, 0x7c0000000000ull);
      Plan* q = nullptr;
      CHECK(cache.prepare(MODE_STEP, s.data(), 1, 3, r, false, &q) == MUON_OK);
    }
    CHECK(cache.stats.evictions == 2);
    CHECK(cache.plan_count() == PlanCache::kMaxPlans + 1);
    Plan* again = nullptr;
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, 3, r0, false, &again) == MUON_OK);
    CHECK(again->key == p0->key || again->ws != old_ws);
  }
  CHECK(ops.live.empty());
}

static void test_caller_workspace() {
  FakeOps ops;
  PlanCache cache(&ops);
  const auto s = gpt2_block(1);
  const auto r = records(s, 0x7f0000000000ull);
  std::vector<char> mine(workspace_bytes_of(s.data(), (int)s.size()) - 256);
  CHECK(cache.set_workspace(mine.data(), mine.size()) == MUON_OK);
  Plan* p = nullptr;
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, r, false, &p) == MUON_ENOMEM);
  std::vector<char> enough(workspace_bytes_of(s.data(), (int)s.size()));
  CHECK(cache.set_workspace(enough.data(), enough.size()) == MUON_OK);
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, r, false, &p) == MUON_OK);
  CHECK(p->ws == enough.data());
  check_tables(*p, s, enough.size());
  cache.release_all();  // does not free the caller's workspace
  CHECK(ops.live.empty());
  ops.fail_alloc = true;
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), 3, r, false, &p) == MUON_ENOMEM);
}

// Lanes regroup the work but never change an item: the same tiles, K
// ranges and partial-tile slots as with one lane.
static void test_lanes_change_no_item() {
  const std::vector<std::vector<muon_shape_t>> sets = {gpt2_block(12), gpt2_block(1),
                                                       shapes_of({{50257, 768}, {768, 768}}),
                                                       shapes_of({{64, 4100}, {512, 20000}, {20001, 300}, {77, 77}})};
  for (const auto& s : sets) {
    std::vector<char> ws(workspace_bytes_of(s.data(), (int)s.size()));
    std::set<std::tuple<int, int, int, int, int, int, int>> items[5];
    size_t lanes_seen[5] = {0, 0, 0, 0, 0};
    for (int L = 1; L <= kMaxLanes; ++L) {
      PlanTables t;
      CHECK(build_tables(MODE_STEP, s.data(), (int)s.size(), ws.data(), L, &t) == MUON_OK);
      lanes_seen[L] = t.lanes.size();
      std::set<std::tuple<int, int, int, int, int, int, int>> got;
      for (const LaneTables& lt : t.lanes) {
        const size_t offs[3] = {lt.o_gram, lt.o_poly, lt.o_upd};
        const int cnts[3] = {lt.n_gram, lt.n_poly, lt.n_upd};
        for (int kind = 0; kind < 3; ++kind) {
          const GemmItem* it = reinterpret_cast<const GemmItem*>(t.image.data() + offs[kind]);
          for (int k = 0; k < cnts[kind]; ++k)
            if (it[k].mat >= 0) got.insert({kind, it[k].mat, it[k].ti, it[k].tj, it[k].k0, it[k].kn, it[k].slot});
        }
      }
      items[L] = got;
      if (L > 1) CHECK(items[L] == items[1]);
    }
    CHECK(lanes_seen[1] == 1);
  }
  // the GPT-2-124M hidden set: three shape groups, three lanes (two with two)
  const auto s = gpt2_block(12);
  const std::vector<int> l3 = lane_of_matrices(s.data(), (int)s.size(), 3);
  const std::vector<int> l2 = lane_of_matrices(s.data(), (int)s.size(), 2);
  CHECK(*std::max_element(l3.begin(), l3.end()) == 2 && *std::max_element(l2.begin(), l2.end()) == 1);
  CHECK(l3[2] == 0 && l3[3] == 0);  // 768 x 3072 and its transpose: the costliest group first
  // small calls: one 256 x 512 matrix (4 update tiles), 1024 x 1536 (36,
  // Gram K 24 slices), 768 x 2048 (32, K 32); not 768 x 2304 (36 tiles but
  // K 36 slices), 256 x 4096 (32 tiles, K 64), one GPT-2 block (144), 768 x
  // 3072 (48), the hidden set (1728), the stress pair (800)
  const auto c1 = shapes_of({{256, 512}}), c5 = shapes_of({{50257, 768}, {768, 768}});
  const auto m36 = shapes_of({{1024, 1536}}), k32 = shapes_of({{768, 2048}}), m48 = shapes_of({{3072, 768}});
  const auto k36 = shapes_of({{768, 2304}}), k64 = shapes_of({{256, 4096}});
  CHECK(small_call(c1.data(), 1) && small_call(m36.data(), 1) && small_call(k32.data(), 1) && !small_call(m48.data(), 1));
  CHECK(!small_call(k36.data(), 1) && !small_call(k64.data(), 1));
  CHECK(!small_call(gpt2_block(1).data(), 4) && !small_call(s.data(), (int)s.size()) && !small_call(c5.data(), 2));
}

// The elementwise passes' block -> item map: a permutation of the items for
// any grid, the identity for runs of one, and in every whole group of 8R
// blocks the blocks of one XCD (b % 8) take R consecutive items.
static void test_elementwise_item_map() {
  const int grids[] = {1, 5, 8, 9, 63, 64, 65, 431, 1000, 5184, 90001};
  const int runs[] = {1, 2, EW_MOM_RUN, EW_TILE_RUN, 64};
  for (int nb : grids)
    for (int run : runs) {
      std::vector<int> seen(nb, 0);
      bool in_range = true;
      for (int b = 0; b < nb; ++b) {
        const int it = ew_item_of_block(b, nb, run);
        if (it < 0 || it >= nb) { in_range = false; continue; }
        ++seen[it];
      }
      CHECK(in_range);
      CHECK(std::all_of(seen.begin(), seen.end(), [](int c) { return c == 1; }));
      if (run == 1)
        for (int b = 0; b < nb; ++b) CHECK(ew_item_of_block(b, nb, 1) == b);
      const int group = 8 * run;
      for (int b = 0; b + group <= nb && b < 4 * group; ++b) {
        const int g = b / group, w = b % group;
        CHECK(ew_item_of_block(b, nb, run) == g * group + (w % 8) * run + w / 8);
      }
    }
}

// Update tiles of the named sets: the medium (128 x 256) tiles where their
// rounds over the CUs cost less than the large tiles' (one GPT-2 block: 216
// against 144 tiles, one round each; two blocks: 432 / 288, two rounds each;
// the stress pair: 1200 / 800, five rounds against four), the large ones
// where they do not (four blocks: 864 / 576, four rounds against three; the
// hidden set: 2592 / 1728, eleven against seven).
static void test_update_tile_choice() {
  const auto c5 = shapes_of({{50257, 768}, {768, 768}});
  CHECK(tile_choice(gpt2_block(1).data(), 4).upd == TILE_MEDIUM);
  // at most 128 medium update tiles: the small tiles with the shallow ring
  // (one 768 x 3072 matrix: 72 medium tiles; 2048 x 2048: 128; 2048 x 3072:
  // 192 stays medium)
  const auto k3 = shapes_of({{768, 3072}}), s2k = shapes_of({{2048, 2048}}), s23 = shapes_of({{2048, 3072}});
  CHECK(tile_choice(k3.data(), 1).upd == TILE_SHALLOW && tile_choice(s2k.data(), 1).upd == TILE_SHALLOW);
  CHECK(tile_choice(s23.data(), 1).upd == TILE_MEDIUM);
  CHECK(tile_choice(gpt2_block(2).data(), 8).upd == TILE_MEDIUM);
  CHECK(tile_choice(c5.data(), 2).upd == TILE_MEDIUM);
  CHECK(tile_choice(gpt2_block(4).data(), 16).upd == TILE_LARGE);
  CHECK(tile_choice(gpt2_block(12).data(), 48).upd == TILE_LARGE);
}

int main() {
  test_elementwise_item_map();
  test_update_tile_choice();
  test_lanes_change_no_item();
  test_validation();
  test_tables_of_many_shapes();
  test_pointer_alternation_needs_no_rebuild();
  test_eviction_and_capture();
  test_caller_workspace();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
