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
    apply += (int64_t)((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE);
  }
  std::sort(regions.begin(), regions.end());
  for (size_t k = 1; k < regions.size(); ++k) CHECK(regions[k].first >= regions[k - 1].second);
  CHECK(t.n_mom == mom && t.n_cast == cast && t.n_apply == apply);
  // elementwise items: each (matrix, index) once, indices in range
  auto ew = [&](size_t off, int cnt, int which) {
    const EwItem* it = p.at<EwItem>(off);
    std::set<std::pair<int, int>> seen;
    for (int k = 0; k < cnt; ++k) {
      CHECK(it[k].mat >= 0 && it[k].mat < n);
      if (it[k].mat < 0 || it[k].mat >= n) continue;
      const Geometry g = geometry_of(s[it[k].mat]);
      const int lim = which == 0 ? g.part_cnt
                      : which == 1 ? (g.m_pad / CAST_TILE) * (g.n_pad / CAST_TILE)
                                   : ((g.rows + CAST_TILE - 1) / CAST_TILE) * ((g.cols + CAST_TILE - 1) / CAST_TILE);
      CHECK(it[k].idx >= 0 && it[k].idx < lim);
      CHECK(seen.insert({it[k].mat, it[k].idx}).second);
    }
  };
  ew(t.o_mom, t.n_mom, 0);
  ew(t.o_cast, t.n_cast, 1);
  ew(t.o_apply, t.n_apply, 2);
  // GEMM items: tiles inside the padded matrix, K ranges inside the true
  // size, each output tile covered once per kind (Gram chunks tile K)
  auto gemm = [&](size_t off, int cnt, int kind) {
    const GemmItem* it = p.at<GemmItem>(off);
    CHECK(cnt % 8 == 0);
    std::map<std::tuple<int, int, int>, int64_t> ksum;
    for (int k = 0; k < cnt; ++k) {
      if (it[k].mat < 0) continue;
      CHECK(it[k].mat < n);
      const MatDesc& m = d[it[k].mat];
      if (kind == 0) {
        CHECK(it[k].ti <= it[k].tj && (it[k].tj + 1) * GRAM_BM <= m.m_pad);
        CHECK(it[k].k0 >= 0 && (int64_t)(it[k].k0 + it[k].kn) * 64 <= m.n_pad && it[k].kn >= 1);
        ksum[{it[k].mat, it[k].ti, it[k].tj}] += it[k].kn;
      } else if (kind == 1) {
        CHECK(it[k].ti <= it[k].tj && (it[k].tj + 1) * SYM_BM <= m.m_pad && it[k].kn * 64 <= m.m_pad);
        ksum[{it[k].mat, it[k].ti, it[k].tj}] += 1;
      } else {
        CHECK(it[k].ti * UPD_ROWU < m.m_pad && (it[k].tj + 1) * UPD_BN <= m.n_pad);
        CHECK(it[k].kn % 2 == 0 && it[k].kn * 64 <= m.m_pad);
        CHECK(it[k].ti * UPD_ROWU + UPD_BM <= m.m_pad + NS_PAD_M);  // overhang inside the spare rows
        ksum[{it[k].mat, it[k].ti, it[k].tj}] += 1;
      }
    }
    for (auto& kv : ksum) {
      const MatDesc& m = d[std::get<0>(kv.first)];
      if (kind == 0) CHECK(kv.second == ((int64_t)m.n + 63) / 64);
      else CHECK(kv.second == 1);
    }
    if (kind == 1) {
      int64_t want = 0;
      for (int i = 0; i < n; ++i) want += (int64_t)(d[i].m_pad / SYM_BM) * (d[i].m_pad / SYM_BM + 1) / 2;
      CHECK((int64_t)ksum.size() == want);
    }
  };
  gemm(t.o_gram, t.n_gram, 0);
  gemm(t.o_poly, t.n_poly, 1);
  gemm(t.o_upd, t.n_upd, 2);
  // partial tiles of cut Gram tiles lie inside the workspace
  const GemmItem* g = p.at<GemmItem>(t.o_gram);
  for (int k = 0; k < t.n_gram; ++k)
    if (g[k].mat >= 0 && g[k].slot >= 0) {
      const char* lo = p.ws + t.gram_part_off + (size_t)g[k].slot * GRAM_BM * GRAM_BM * 4;
      CHECK(lo >= p.ws && lo + GRAM_BM * GRAM_BM * 4 <= ws_hi);
    }
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
      CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), r, false, &p) == MUON_OK);
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
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), a, false, &p) == MUON_OK);
  const CacheStats first = cache.stats;
  CHECK(first.plan_builds == 1 && first.uploads == 1 && first.syncs == 0 && first.ws_allocs == 1);
  CHECK(first.patch_calls == 2);  // 48 matrices, 40 per patch
  // the same pointers again: nothing but the launches
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), a, false, &p) == MUON_OK);
  CHECK(cache.stats.patch_calls == first.patch_calls);
  for (int k = 0; k < 10; ++k) {
    const auto& r = (k % 2) ? a : b;
    Plan* q = nullptr;
    CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), r, false, &q) == MUON_OK);
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
  CHECK(cache.prepare(MODE_NS, s.data(), (int)s.size(), x, false, &p) == MUON_OK);
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
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, r0, true, &p0) == MUON_EINVAL);  // never seen: refused
    CHECK(cache.stats.plan_builds == 0);
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, r0, false, &p0) == MUON_OK);
    const int64_t before = cache.stats.patch_calls;
    Plan* pc = nullptr;
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, r0, true, &pc) == MUON_OK);
    CHECK(pc == p0 && pc->captured);
    CHECK(cache.stats.patch_calls == before + 1);  // a capture always records the pointer write
    // eager calls on a captured plan always re-patch (a replay writes its own pointers)
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, r0, false, &pc) == MUON_OK);
    CHECK(cache.stats.patch_calls == before + 2);
    // a larger set of shapes refused under capture (it would allocate)
    const auto big = gpt2_block(1);
    const auto rb = records(big, 0x7d0000000000ull);
    Plan* pb = nullptr;
    CHECK(cache.prepare(MODE_STEP, big.data(), (int)big.size(), rb, true, &pb) == MUON_EINVAL);
    // ... fine eagerly: the workspace grows, the captured plan keeps the old one
    char* old_ws = p0->ws;
    CHECK(cache.prepare(MODE_STEP, big.data(), (int)big.size(), rb, false, &pb) == MUON_OK);
    CHECK(cache.stats.syncs == 1);
    CHECK(ops.live.count(old_ws) == 1);  // retired, not freed
    CHECK(p0->captured && p0->ws == old_ws);
    // nine more shape sets: uncaptured plans are evicted, the captured one stays
    for (int k = 0; k < 9; ++k) {
      const auto s = shapes_of({{32 + k, 48}});
      const auto r = records(s, 0x7c0000000000ull);
      Plan* q = nullptr;
      CHECK(cache.prepare(MODE_STEP, s.data(), 1, r, false, &q) == MUON_OK);
    }
    CHECK(cache.stats.evictions == 2);
    CHECK(cache.plan_count() == PlanCache::kMaxPlans + 1);
    Plan* again = nullptr;
    CHECK(cache.prepare(MODE_STEP, s0.data(), 1, r0, false, &again) == MUON_OK);
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
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), r, false, &p) == MUON_ENOMEM);
  std::vector<char> enough(workspace_bytes_of(s.data(), (int)s.size()));
  CHECK(cache.set_workspace(enough.data(), enough.size()) == MUON_OK);
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), r, false, &p) == MUON_OK);
  CHECK(p->ws == enough.data());
  check_tables(*p, s, enough.size());
  cache.release_all();  // does not free the caller's workspace
  CHECK(ops.live.empty());
  ops.fail_alloc = true;
  CHECK(cache.prepare(MODE_STEP, s.data(), (int)s.size(), r, false, &p) == MUON_ENOMEM);
}

int main() {
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
