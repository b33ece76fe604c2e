// C ABI of the Muon step library: the HIP side of the plan cache (device
// table blocks, workspace, stream-ordered uploads and pointer patches) and
// the launch sequence.  Validation, geometry and the table images are plain host code
// in plan_host.cpp.  The operation itself is described in include/muon.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/muon.h"
#include "api_internal.h"
#include "muon_internal.h"
#include "plan_host.h"

namespace muon {

int fail_hip(hipError_t e, const char* what) { return fail(MUON_EHIP, "%s: %s", what, hipGetErrorString(e)); }

std::mutex& api_mutex() {
  static std::mutex mu;
  return mu;
}

namespace {

// DeviceOps over HIP, in the order of the current call's stream.
class HipOps : public DeviceOps {
 public:
  hipStream_t stream = nullptr;

  int alloc_tables(size_t bytes, void** dev, void** host) override {
    *dev = *host = nullptr;
    hipError_t e = hipHostMalloc(host, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      *host = nullptr;
      (void)hipGetLastError();
      return fail(MUON_ENOMEM, "hipHostMalloc of %zu plan bytes failed: %s", bytes, hipGetErrorString(e));
    }
    if ((e = hipMalloc(dev, bytes)) != hipSuccess) {
      *dev = nullptr;
      (void)hipGetLastError();
      (void)hipHostFree(*host);
      *host = nullptr;
      return fail(MUON_ENOMEM, "hipMalloc of %zu plan bytes failed: %s", bytes, hipGetErrorString(e));
    }
    return MUON_OK;
  }
  void free_tables(void* dev, void* host) override {
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
  }
  int upload(void* dev, void* host, const void* image, size_t bytes) override {
    memcpy(host, image, bytes);
    const hipError_t e = hipMemcpyAsync(dev, host, bytes, hipMemcpyHostToDevice, stream);
    return e == hipSuccess ? MUON_OK : fail_hip(e, "hipMemcpyAsync(plan tables)");
  }
  int patch(void* dev_desc, const PtrRecord* recs, int count) override {
    return patch_records(static_cast<MatDesc*>(dev_desc), std::vector<PtrRecord>(recs, recs + count), stream);
  }
  int alloc_workspace(size_t bytes, void** p) override {
    const char* inject = getenv("MUON_TEST_FAIL_ALLOC");
    if (inject && inject[0] == '1') return fail(MUON_ENOMEM, "workspace allocation of %zu bytes failed (injected)", bytes);
    const hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      *p = nullptr;
      (void)hipGetLastError();
      return fail(MUON_ENOMEM, "hipMalloc of %zu workspace bytes failed: %s", bytes, hipGetErrorString(e));
    }
    return MUON_OK;
  }
  void free_workspace(void* p) override {
    if (p) (void)hipFree(p);
  }
  int sync_device() override {
    const hipError_t e = hipDeviceSynchronize();
    return e == hipSuccess ? MUON_OK : fail_hip(e, "hipDeviceSynchronize");
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
  bool captured = false;
  ~AdamPlan() {
    if (dev) (void)hipFree(dev);
    if (host) (void)hipHostFree(host);
  }
};

// Internal streams of a device's lanes, and the events that fork them from
// and join them to the caller's stream.  Created on the first call with more
// than one lane; default priority, non-blocking (ordered only by the events).
struct LaneStreams {
  bool ready = false;
  hipStream_t s[kMaxLanes] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kMaxLanes] = {};

  int create() {
    if (ready) return MUON_OK;
    hipError_t e;
    for (int l = 0; l < kMaxLanes; ++l) {
      if ((e = hipStreamCreateWithFlags(&s[l], hipStreamNonBlocking)) != hipSuccess) return fail_hip(e, "hipStreamCreateWithFlags");
      if ((e = hipEventCreateWithFlags(&join[l], hipEventDisableTiming)) != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    }
    if ((e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) != hipSuccess) return fail_hip(e, "hipEventCreateWithFlags");
    ready = true;
    return MUON_OK;
  }
  void destroy() {
    for (int l = 0; l < kMaxLanes; ++l) {
      if (s[l]) (void)hipStreamDestroy(s[l]);
      if (join[l]) (void)hipEventDestroy(join[l]);
      s[l] = nullptr;
      join[l] = nullptr;
    }
    if (fork) (void)hipEventDestroy(fork);
    fork = nullptr;
    ready = false;
  }
};

struct DeviceState {
  HipOps ops;
  PlanCache cache{&ops};
  std::list<std::unique_ptr<AdamPlan>> adam_plans;  // most recent first
  LaneStreams lanes;
};

int g_max_lanes = kDefaultLanes;

std::map<int, std::unique_ptr<DeviceState>> g_dev;
constexpr size_t kMaxAdamPlans = 8;

DeviceState& device_state(int dev) {
  auto& p = g_dev[dev];
  if (!p) p = std::make_unique<DeviceState>();
  return *p;
}

}  // namespace

// Timing of one kernel family (muon_timing_enable).
int g_time_kind = -1;
std::vector<hipEvent_t> g_ev;  // start, end pairs
size_t g_ev_used = 0;

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

int capture_status(hipStream_t stream, bool* capturing) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return fail_hip(e, "hipStreamIsCapturing");
  *capturing = cs != hipStreamCaptureStatusNone;
  return MUON_OK;
}

Tables tables_at(char* block, const PlanTables& t, int lane, char* ws) {
  const LaneTables& lt = t.lanes[lane];
  Tables v;
  v.desc = reinterpret_cast<MatDesc*>(block + t.o_desc);
  v.mats = reinterpret_cast<int32_t*>(block + lt.o_mats);
  v.fin = reinterpret_cast<int32_t*>(block + lt.o_fin);
  v.mom = reinterpret_cast<EwItem*>(block + lt.o_mom);
  v.cast = reinterpret_cast<EwItem*>(block + lt.o_cast);
  v.apply = reinterpret_cast<EwItem*>(block + lt.o_apply);
  v.gram = reinterpret_cast<GemmItem*>(block + lt.o_gram);
  v.poly = reinterpret_cast<GemmItem*>(block + lt.o_poly);
  v.upd = reinterpret_cast<GemmItem*>(block + lt.o_upd);
  v.red = reinterpret_cast<RedItem*>(block + lt.o_red);
  v.gram_part = reinterpret_cast<float*>(ws + t.gram_part_off);
  v.small = t.small;
  v.fused = t.fused;
  v.gram_tile = t.gram_tile;
  v.poly_tile = t.poly_tile;
  v.upd_tile = t.upd_tile;
  v.gram_bm = t.gram_bm;
  v.t = &lt;
  return v;
}

// The kernel sequence of one lane: momentum and norm, cast, ns_steps
// iterations of Gram, poly and update, apply.
int launch_sequence(int mode, const Tables& v, float lr, float beta, int ns_steps, const float* coeffs, int stride,
                    hipStream_t stream) {
  const LaneTables& t = *v.t;
  int rc;
  if (mode == MODE_STEP) {
    rc = timed(MUON_KERNEL_MOMENTUM, stream,
               [&] { return launch_momentum(v.desc, v.mom, t.n_mom, v.fin, t.n_fin, beta, stream); },
               "momentum kernel launch");
    if (rc) return rc;
  }
  rc = timed(MUON_KERNEL_CAST, stream, [&] { return launch_cast(v.desc, v.cast, t.n_cast, beta, mode == MODE_NS, stream); },
             "cast kernel launch");
  if (rc) return rc;
  for (int k = 0; k < ns_steps; ++k) {
    const int src = k & 1;
    const float* ck = coeffs + (size_t)k * stride;  // iteration k's a, b, c
    const float ca = ck[0], cb = ck[1], cc = ck[2];
    rc = timed(MUON_KERNEL_GRAM, stream,
               [&] {
                 const hipError_t e = launch_gemm(GEMM_GRAM, v.desc, v.gram, t.n_gram, src, ca, cb, cc, v.gram_part, v.gram_tile, stream);
                 return e != hipSuccess ? e : launch_gram_reduce(v.desc, v.red, t.n_red, v.gram_part, v.gram_bm, stream);
               },
               "gram kernel launch");
    if (rc) return rc;
    if (v.fused) {
      // poly and update in one launch (timed as the update)
      rc = timed(MUON_KERNEL_UPDATE, stream,
                 [&] { return launch_poly_update(v.desc, v.upd, t.n_upd, src, ca, cb, cc, stream); },
                 "poly-update kernel launch");
      if (rc) return rc;
      continue;
    }
    rc = timed(MUON_KERNEL_POLY, stream,
               [&] { return launch_gemm(GEMM_POLY, v.desc, v.poly, t.n_poly, src, ca, cb, cc, nullptr, v.poly_tile, stream); },
               "poly kernel launch");
    if (rc) return rc;
    rc = timed(MUON_KERNEL_UPDATE, stream,
               [&] { return launch_gemm(GEMM_UPDATE, v.desc, v.upd, t.n_upd, src, ca, cb, cc, nullptr, v.upd_tile, stream); },
               "update kernel launch");
    if (rc) return rc;
  }
  return timed(MUON_KERNEL_APPLY, stream,
               [&] { return launch_apply(v.desc, v.apply, t.n_apply, lr, ns_steps & 1, mode == MODE_STEP, stream); },
               "apply kernel launch");
}

int patch_records(MatDesc* desc, const std::vector<PtrRecord>& recs, hipStream_t stream) {
  const int n = (int)recs.size();
  for (int i = 0; i < n; i += PATCH_MAX) {
    PtrPatch p{};
    p.count = std::min(PATCH_MAX, n - i);
    for (int k = 0; k < p.count; ++k) p.rec[k] = recs[i + k];
    const hipError_t e = launch_ptr_patch(desc, p, stream);
    if (e != hipSuccess) return fail_hip(e, "pointer patch launch");
  }
  return MUON_OK;
}

namespace {

int run(int mode, float* const* params, const float* const* grads, float* const* moms, uint16_t* const* upd,
        const uint16_t* const* xin, const muon_shape_t* shapes, int n, float lr, float beta, int ns_steps,
        const float* coeffs, int stride, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  bool capturing = false;
  int rc = capture_status(stream, &capturing);
  if (rc) return rc;
  std::vector<PtrRecord> recs;
  make_ptr_records(mode, shapes, n, params, grads, moms, upd, xin, &recs);
  std::lock_guard<std::mutex> lock(api_mutex());
  DeviceState& st = device_state(dev);
  st.ops.stream = stream;
  Plan* p = nullptr;
  if ((rc = st.cache.prepare(mode, shapes, n, g_max_lanes, recs, capturing, &p))) return rc;
  char* block = static_cast<char*>(p->dev);
  const int L = (int)p->t.lanes.size();
  if (L == 1 || capturing) {
    // one lane, or under capture: every lane in turn on the caller's stream
    for (int l = 0; l < L; ++l)
      if ((rc = launch_sequence(mode, tables_at(block, p->t, l, p->ws), lr, beta, ns_steps, coeffs, stride, stream)))
        return rc;
    return MUON_OK;
  }
  // Several lanes: each runs its matrices' whole step on its own stream,
  // after everything the caller enqueued before (the pointer patches
  // included), and the caller's stream continues once all have finished.
  LaneStreams& ls = st.lanes;
  if ((rc = ls.create())) return rc;
  if ((e = hipEventRecord(ls.fork, stream)) != hipSuccess) return fail_hip(e, "hipEventRecord(fork)");
  for (int l = 0; l < L; ++l) {
    if ((e = hipStreamWaitEvent(ls.s[l], ls.fork, 0)) != hipSuccess) return fail_hip(e, "hipStreamWaitEvent(fork)");
    if ((rc = launch_sequence(mode, tables_at(block, p->t, l, p->ws), lr, beta, ns_steps, coeffs, stride, ls.s[l])))
      return rc;
    if ((e = hipEventRecord(ls.join[l], ls.s[l])) != hipSuccess) return fail_hip(e, "hipEventRecord(join)");
  }
  for (int l = 0; l < L; ++l)
    if ((e = hipStreamWaitEvent(stream, ls.join[l], 0)) != hipSuccess) return fail_hip(e, "hipStreamWaitEvent(join)");
  return MUON_OK;
}

int step_entry(float* const* params, const float* const* grads, float* const* momentum, const muon_shape_t* shapes,
               int n, float lr, float beta, int ns_steps, const float* coeffs, int stride, uint16_t* const* updates,
               hipStream_t stream) {
  clear_error();
  int rc = validate_step(params, grads, momentum, shapes, n, lr, beta, ns_steps, coeffs, stride, updates);
  if (rc || n == 0) return rc;
  return run(MODE_STEP, params, grads, momentum, updates, nullptr, shapes, n, lr, beta, ns_steps, coeffs, stride,
             stream);
}

int ns_entry(const uint16_t* const* x, uint16_t* const* out, const muon_shape_t* shapes, int n, int ns_steps,
             const float* coeffs, int stride, hipStream_t stream) {
  clear_error();
  int rc = validate_ns(x, out, shapes, n, ns_steps, coeffs, stride);
  if (rc || n == 0) return rc;
  return run(MODE_NS, nullptr, nullptr, nullptr, out, x, shapes, n, 0.0f, 0.0f, ns_steps, coeffs, stride, stream);
}

// ---------------------------------------------------------------- AdamW ----

// wd[i] is a tensor's own lambda, baked into the plan, unless shared[i] is
// set: then the call's shared lambda (a kernel argument) applies.  The shared
// lambda can change from call to call (a weight-decay schedule) without a new
// plan.  A plan built outside capture and then used under capture is kept
// until release (a graph reads its tables).
int get_adam_plan(DeviceState& st, int n, float* const* params, const float* const* grads, float* const* u,
                  float* const* v, const int64_t* numels, const float* wd, const int* shared, bool capturing,
                  hipStream_t stream, AdamPlan** out) {
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
      st.adam_plans.front()->captured |= capturing;
      *out = st.adam_plans.front().get();
      return MUON_OK;
    }
  }
  if (capturing)
    return fail(MUON_EINVAL, "no AdamW plan for these tensors yet: make one call with them before capturing it into a graph");
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
  int rc = st.ops.alloc_tables(bytes, &plan->dev, &plan->host);
  if (rc) return rc;
  char* h = static_cast<char*>(plan->host);
  memcpy(h + o_desc, desc.data(), sizeof(AdamDesc) * n);
  memcpy(h + o_items, items.data(), sizeof(EwItem) * items.size());
  // the pinned staging lives as long as the plan, so the copy needs no wait
  const hipError_t e = hipMemcpyAsync(plan->dev, plan->host, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(adamw plan)");
  plan->d_desc = reinterpret_cast<AdamDesc*>(static_cast<char*>(plan->dev) + o_desc);
  plan->d_items = reinterpret_cast<EwItem*>(static_cast<char*>(plan->dev) + o_items);
  plan->n_items = (int)items.size();
  st.adam_plans.push_front(std::move(plan));
  AdamPlan* fresh = st.adam_plans.front().get();
  size_t uncaptured = 0;
  for (auto& q : st.adam_plans) uncaptured += q->captured ? 0 : 1;
  if (uncaptured > kMaxAdamPlans) {
    // the least recently used uncaptured plan goes once the device is done with it
    for (auto it = std::prev(st.adam_plans.end());; --it) {
      if (!(*it)->captured && it->get() != fresh) {
        if ((rc = st.ops.sync_device())) return rc;
        st.adam_plans.erase(it);
        break;
      }
      if (it == st.adam_plans.begin()) break;
    }
  }
  *out = fresh;
  return MUON_OK;
}

int adamw_entry(float* const* params, const float* const* grads, float* const* u, float* const* v,
                const int64_t* numels, const float* wd, int n, float lr, float beta1, float beta2, float eps,
                int64_t step, hipStream_t stream) {
  clear_error();
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
  bool capturing = false;
  if ((rc = capture_status(stream, &capturing))) return rc;
  std::lock_guard<std::mutex> lock(api_mutex());
  DeviceState& st = device_state(dev);
  st.ops.stream = stream;
  AdamPlan* p = nullptr;
  if ((rc = get_adam_plan(st, (int)P.size(), P.data(), G.data(), U.data(), V.data(), N.data(), W.data(), S.data(),
                          capturing, stream, &p)))
    return rc;
  return timed(MUON_KERNEL_ADAMW, stream, [&] { return launch_adamw(p->d_desc, p->d_items, p->n_items, c, stream); },
               "adamw kernel launch");
}

int untie_entry(const float* const src[3], float* const dst[3], int64_t rows, int64_t cols, int transpose,
                hipStream_t stream) {
  clear_error();
  const int rc = validate_untie(src, dst, rows, cols, transpose);
  if (rc) return rc;
  const size_t b = (size_t)rows * cols * sizeof(float);
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
}  // namespace muon

using namespace muon;

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

const char* muon_last_error(void) { return last_error_text(); }

size_t muon_workspace_bytes(const muon_shape_t* shapes, int n) {
  clear_error();
  if (check_shapes(shapes, n)) return 0;
  return workspace_bytes_of(shapes, n);
}

int muon_set_workspace(void* dev_ptr, size_t bytes) {
  clear_error();
  if ((dev_ptr == nullptr) != (bytes == 0)) return fail(MUON_EINVAL, "dev_ptr and bytes must both be set or both be 0");
  if ((uintptr_t)dev_ptr % kAlign) return fail(MUON_EINVAL, "workspace must be %zu-byte aligned", kAlign);
  if (dev_ptr && bytes < kControlBytes)
    return fail(MUON_ENOMEM, "workspace of %zu bytes is below the %zu-byte minimum", bytes, kControlBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(api_mutex());
  return device_state(dev).cache.set_workspace(dev_ptr, bytes);
}

void muon_release(void) {
  std::lock_guard<std::mutex> lock(api_mutex());
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_dev) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    kv.second->cache.release_all();
    kv.second->adam_plans.clear();
    kv.second->lanes.destroy();
  }
  (void)hipSetDevice(cur);
  g_dev.clear();
  for (hipEvent_t ev : g_ev) (void)hipEventDestroy(ev);
  g_ev.clear();
  g_ev_used = 0;
}

int muon_plan_stats(int64_t out[6]) {
  clear_error();
  if (!out) return fail(MUON_EINVAL, "out must not be NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(api_mutex());
  const CacheStats& s = device_state(dev).cache.stats;
  const int64_t v[6] = {s.plan_builds, s.uploads, s.patch_calls, s.syncs, s.evictions, s.ws_allocs};
  for (int k = 0; k < 6; ++k) out[k] = v[k];
  return MUON_OK;
}

int muon_set_lanes(int lanes) {
  clear_error();
  if (lanes < 1 || lanes > kMaxLanes) return fail(MUON_EINVAL, "lanes = %d outside [1, %d]", lanes, kMaxLanes);
  std::lock_guard<std::mutex> lock(api_mutex());
  g_max_lanes = lanes;
  return MUON_OK;
}

int muon_timing_enable(int kernel) {
  clear_error();
  if (kernel < -1 || kernel > MUON_KERNEL_ADAMW) return fail(MUON_EINVAL, "unknown kernel family %d", kernel);
  std::lock_guard<std::mutex> lock(api_mutex());
  g_time_kind = kernel;
  g_ev_used = 0;
  return MUON_OK;
}

int muon_timing_read(double* total_ms, int64_t* launches) {
  clear_error();
  if (!total_ms || !launches) return fail(MUON_EINVAL, "output pointers must not be NULL");
  std::lock_guard<std::mutex> lock(api_mutex());
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
