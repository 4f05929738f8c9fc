// C entry points of libdmuon_ns: validation, planning, launch sequence, timing.
//
// The step follows the DMuon "架构设计" (Architecture design) page: §1 gives the
// Newton–Schulz equation, §2 says only the owner runs NS + momentum + weight
// decay + parameter update on its local full-precision copy without any
// communication; the HSDP guide ("what happens underneath", step 3) repeats it.
// Rank checks follow the MindSpore parameter-grouping page §2.1 / §4.1 (fewer
// than two dims is an error) and §2.2 / §6 (the matrix is the last two dims).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dmuon_ns.h"
#include "internal.hpp"

namespace dmuon {

static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int lpt_fail(int code, const char* msg) { return fail(code, msg); }
void clear_error() { g_err.clear(); }

// ---------------------------------------------------------------------------
// phase timing (opt-in)
// ---------------------------------------------------------------------------
struct TimedLaunch {
  int phase;
  hipEvent_t a, b;
};
static std::mutex g_tmu;
static bool g_timing = false;
static std::vector<TimedLaunch> g_timed;
static std::vector<hipEvent_t> g_evpool;
static hipEvent_t g_pending = nullptr;

static hipEvent_t take_event() {
  if (!g_evpool.empty()) {
    hipEvent_t e = g_evpool.back();
    g_evpool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void timing_before(int phase, void* stream) {
  (void)phase;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing) return;
  g_pending = take_event();
  if (g_pending) (void)hipEventRecord(g_pending, (hipStream_t)stream);
}

void timing_after(int phase, void* stream) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || !g_pending) return;
  hipEvent_t b = take_event();
  if (!b) return;
  (void)hipEventRecord(b, (hipStream_t)stream);
  g_timed.push_back({phase, g_pending, b});
  g_pending = nullptr;
}

// ---------------------------------------------------------------------------
// table upload through pinned staging
//
// The per-call tensor table is copied host → device on the caller's stream.  A
// copy from pageable memory may hold the host until the stream reaches it, so
// the host could not enqueue ahead of the GPU.  The table is staged instead in
// one of kStaging pinned buffers; an event recorded after each copy tells when
// the buffer may be reused (by then it is long done: kStaging calls later).
// ---------------------------------------------------------------------------
constexpr int kStaging = 8;
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
};
static std::mutex g_smu;
static Staging g_stage[kStaging];
static int g_stage_next = 0;

static int stage_upload(void* dst, const void* src, size_t bytes, void* stream) {
  std::lock_guard<std::mutex> lk(g_smu);
  Staging& st = g_stage[g_stage_next];
  g_stage_next = (g_stage_next + 1) % kStaging;
  hipError_t e;
  if (st.done && (e = hipEventSynchronize(st.done)) != hipSuccess) return (int)e;
  if (st.cap < bytes) {
    if (st.host && (e = hipHostFree(st.host)) != hipSuccess) return (int)e;
    st.host = nullptr;
    st.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 64 << 10);
    if ((e = hipHostMalloc(&st.host, cap, hipHostMallocDefault)) != hipSuccess) return (int)e;
    st.cap = cap;
  }
  std::memcpy(st.host, src, bytes);
  if ((e = hipMemcpyAsync(dst, st.host, bytes, hipMemcpyHostToDevice, (hipStream_t)stream)) != hipSuccess)
    return (int)e;
  if (!st.done && (e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming)) != hipSuccess) return (int)e;
  return (int)hipEventRecord(st.done, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// planning
// ---------------------------------------------------------------------------
struct Item {
  int64_t batch, rows, cols;
  const void* grad;
  int grad_bf16;
  float* mom;
  float* master;
  float* out;
  uint16_t* pub;
};

struct Plan {
  std::vector<DevProblem> probs;
  std::vector<int32_t> prefix;      // PH_COUNT × (n + 1)
  int64_t total_slices = 0;
  int64_t total_wg[PH_COUNT] = {};
  size_t off_prefix = 0, off_scal = 0, table_bytes = 0, bytes = 0;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Lay out the workspace for the items; with base == nullptr only sizes are computed.
static int build_plan(const std::vector<Item>& items, int prec_f32, Plan& pl, char* base) {
  const size_t esz = prec_f32 ? 4 : 2;
  const int n = (int)items.size();
  pl.probs.assign(n, DevProblem{});
  pl.prefix.assign((size_t)PH_COUNT * (n + 1), 0);
  size_t off = align256((size_t)n * sizeof(DevProblem));
  pl.off_prefix = off;
  off = align256(off + pl.prefix.size() * sizeof(int32_t));
  pl.table_bytes = off;
  int64_t slices = 0;
  for (const Item& it : items) slices += it.batch;
  pl.total_slices = slices;
  pl.off_scal = off;
  off = align256(off + (size_t)slices * kScalStride * sizeof(float));

  int64_t wg[PH_COUNT] = {};
  int64_t slice_base = 0;
  auto carve = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off = align256(off + bytes);
    return p;
  };
  // Problems in order of falling contraction length (n, then m; stable), so
  // every phase's grid starts with its longest tiles and the short ones fill in
  // behind them.
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    const int64_t nx = std::max(items[x].rows, items[x].cols), ny = std::max(items[y].rows, items[y].cols);
    if (nx != ny) return nx > ny;
    return std::min(items[x].rows, items[x].cols) > std::min(items[y].rows, items[y].cols);
  });
  for (int i = 0; i < n; ++i) {
    const Item& it = items[order[i]];
    DevProblem& P = pl.probs[i];
    P.batch = (int32_t)it.batch;
    P.rows = (int32_t)it.rows;
    P.cols = (int32_t)it.cols;
    P.wide = it.rows <= it.cols ? 1 : 0;
    P.m = (int32_t)std::min(it.rows, it.cols);
    P.n = (int32_t)std::max(it.rows, it.cols);
    P.ld_m = (int32_t)round_up(P.m, kLdAlign);
    P.ld_n = (int32_t)round_up(P.n, kLdAlign);
    P.grad_bf16 = it.grad_bf16;
    const int64_t per = it.rows * it.cols;
    P.chunks = (int32_t)cdiv(per, kElemChunk);
    P.prep_tiles_r = (int32_t)cdiv(it.rows, kPrepTile);
    P.prep_tiles_c = (int32_t)cdiv(it.cols, kPrepTile);
    P.tiles_m = (int32_t)cdiv(P.m, kTile);
    P.apply_tr = (int32_t)cdiv(it.rows, kTile);
    P.apply_tc = (int32_t)cdiv(it.cols, kTile);
    P.slice_base = (int32_t)slice_base;
    P.ld_x = (int32_t)round_up(it.cols, 32);   // 128-byte rows
    slice_base += it.batch;
    P.grad = it.grad;
    P.mom = it.mom;
    P.master = it.master;
    P.out = it.out;
    P.pub = it.pub;
    const int64_t b = it.batch;
    const int64_t prep = (int64_t)P.prep_tiles_r * P.prep_tiles_c;
    // the iterate: 24-bit values (3 bytes) on the bf16 path, fp32 on the fp32 path
    P.xf = (float*)carve((size_t)(b * P.apply_tr * P.apply_tc) * kTile * kTile * (prec_f32 ? 4 : 3));
    if (!it.mom) P.xraw = (float*)carve((size_t)(b * it.rows * P.ld_x) * 4);
    if (prec_f32) {
      P.xg = carve((size_t)(b * P.m * P.ld_n) * esz);
      P.xa0 = carve((size_t)(b * P.n * P.ld_m) * esz);
      P.xa1 = carve((size_t)(b * P.n * P.ld_m) * esz);
    } else {
      const int64_t ld_s = round_up(it.cols, kLdAlign);
      P.xs[0] = carve((size_t)(b * it.rows * ld_s) * esz);
      P.xs[1] = carve((size_t)(b * it.rows * ld_s) * esz);
    }
    P.ap = carve((size_t)(b * P.m * P.ld_m) * esz);
    P.bp = carve((size_t)(b * P.m * P.ld_m) * esz);
    P.part_norm = (float*)carve((size_t)(b * prep) * 4);
    P.x0 = it.mom ? it.mom : P.xraw;
    P.ld_x0 = it.mom ? (int32_t)it.cols : P.ld_x;
    P.part_apply = (float*)carve((size_t)(b * P.apply_tr * P.apply_tc) * 4);
    const int64_t tri = (int64_t)P.tiles_m * (P.tiles_m + 1) / 2;
    const int64_t cnt[PH_COUNT] = {b * prep, b, b * tri, b * tri, b * P.apply_tr * P.apply_tc, b * P.chunks, 0, 0};
    for (int ph = 0; ph < PH_COUNT; ++ph) {
      P.wg0[ph] = (int32_t)wg[ph];
      pl.prefix[(size_t)ph * (n + 1) + i] = (int32_t)wg[ph];
      wg[ph] += cnt[ph];
      if (wg[ph] > INT32_MAX) return fail(DMUON_E_SHAPE, "too many workgroups in one launch");
    }
  }
  for (int ph = 0; ph < PH_COUNT; ++ph) {
    pl.prefix[(size_t)ph * (n + 1) + n] = (int32_t)wg[ph];
    pl.total_wg[ph] = wg[ph];
  }
  pl.bytes = off;
  return DMUON_OK;
}

static int run_plan(Plan& pl, char* ws, int prec_f32, const LaunchScalars& base_s, int steps, void* stream) {
  // descriptors + prefix arrays: one host → device copy, ordered on the stream
  std::vector<char> host(pl.table_bytes, 0);
  std::memcpy(host.data(), pl.probs.data(), pl.probs.size() * sizeof(DevProblem));
  std::memcpy(host.data() + pl.off_prefix, pl.prefix.data(), pl.prefix.size() * sizeof(int32_t));
  int e = stage_upload(ws, host.data(), host.size(), stream);
  if (e) return fail(DMUON_E_HIP, std::string("table upload: ") + hip_error_string(e));
  LaunchTable tab;
  tab.probs = (const DevProblem*)ws;
  tab.wg_prefix = (const int32_t*)(ws + pl.off_prefix);
  tab.scal = (float*)(ws + pl.off_scal);
  tab.n_probs = (int32_t)pl.probs.size();
  auto go = [&](int ph, const LaunchScalars& s) -> int {
    tab.total_wg = (int32_t)pl.total_wg[ph];
    const int r = launch_phase(ph, prec_f32, tab, s, stream);
    if (r) return fail(DMUON_E_HIP, std::string("launch failed: ") + hip_error_string(r));
    return DMUON_OK;
  };
  LaunchScalars s = base_s;
  s.t = 0;
  s.last = 0;
  if ((e = go(PH_INGEST, s))) return e;
  if ((e = go(PH_NORM, s))) return e;
  if (steps == 0) return go(PH_UPDATE, s);
  for (int t = 0; t < steps; ++t) {
    s.t = t;
    s.last = t == steps - 1;
    if ((e = go(PH_GRAM, s))) return e;
    if ((e = go(PH_SQUARE, s))) return e;
    if ((e = go(PH_APPLY, s))) return e;
  }
  return DMUON_OK;
}

// ---------------------------------------------------------------------------
// concurrent groups
//
// Every phase launch ends with a partly filled round of tiles, and the next
// phase of the same tensors cannot start before it ends.  The tensors are
// therefore split into work-balanced groups (greedy largest-first over an
// estimate of each tensor's contraction work), each with its own table and
// launch sequence; group 0 runs on the caller's stream and the others on
// library streams forked from it and joined back with events, so one group's
// tail rounds overlap another group's next phase.  Each slice's arithmetic is
// the same whatever its group, so results do not depend on the split.
// ---------------------------------------------------------------------------
constexpr int kMaxGroups = 4;

// Group count from the rounds of apply tiles on the 256 CUs of an MI355X (a
// fixed count keeps the workspace size a host-only computation).  Measured, ms
// per step with 1 / 2 / 3 / 4 groups:
// * below 4 rounds: four groups, whose tail rounds and epilogues overlap each
//   other's contractions (one d=2048 layer: 2.61 / 2.46 / 2.47 / 2.42);
// * otherwise one: the tails are a small share, and one launch sequence keeps
//   the operand panels of neighbouring tiles together in each XCD's L2 (Llama
//   d=4096 share: 58.2 / 60.2; MLP/MoE mix of 8192-wide matrices and 1408-wide
//   experts: 116.1 / 122.0; 384 small matrices: 2.74 / 2.76).
constexpr int kCusAssumed = 256;

static int group_count(const std::vector<Item>& items) {
  double tiles = 0;
  for (const Item& it : items) tiles += (double)it.batch * cdiv(it.rows, kTile) * cdiv(it.cols, kTile);
  int g = tiles < 4.0 * kCusAssumed ? 4 : 1;
  if (const char* v = std::getenv("DMUON_STREAM_GROUPS")) {   // tuning override, 1..4
    const int x = std::atoi(v);
    if (x >= 1 && x <= kMaxGroups) g = x;
  }
  return std::min<int>(g, (int)items.size());
}

static double item_cost(const Item& it) {
  const int64_t m = std::min(it.rows, it.cols), n = std::max(it.rows, it.cols);
  const int64_t T = cdiv(m, kTile), tri = T * (T + 1) / 2;
  const int64_t app = cdiv(it.rows, kTile) * cdiv(it.cols, kTile);
  const double km = (double)round_up(m, kLdAlign), kn = (double)round_up(n, kLdAlign);
  return (double)it.batch * ((double)tri * kn + (double)tri * km + (double)app * km);
}

struct GroupPlan {
  std::vector<Plan> plans;
  std::vector<size_t> offs;
  size_t bytes = 0;
};

// Split the items, size (base == nullptr) or lay out every group's plan.
static int plan_groups(const std::vector<Item>& items, int prec_f32, char* base, GroupPlan& gp) {
  const int G = group_count(items);
  std::vector<std::vector<Item>> groups(G);
  std::vector<int> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return item_cost(items[x]) > item_cost(items[y]); });
  std::vector<double> load(G, 0.0);
  for (int idx : order) {
    int g = 0;
    for (int k = 1; k < G; ++k)
      if (load[k] < load[g]) g = k;
    groups[g].push_back(items[idx]);
    load[g] += item_cost(items[idx]);
  }
  gp.plans.assign(G, Plan{});
  gp.offs.assign(G, 0);
  size_t off = 0;
  for (int g = 0; g < G; ++g) {
    int e = build_plan(groups[g], prec_f32, gp.plans[g], nullptr);
    if (e) return e;
    gp.offs[g] = off;
    off = align256(off + gp.plans[g].bytes);
    if (base && (e = build_plan(groups[g], prec_f32, gp.plans[g], base + gp.offs[g]))) return e;
  }
  gp.bytes = off;
  return DMUON_OK;
}

struct DeviceStreams {
  hipStream_t s[kMaxGroups - 1] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kMaxGroups - 1] = {};
  std::mutex mu;
};
static std::mutex g_dsmu;
static std::vector<DeviceStreams*> g_ds;

// Library streams and events of the current device (created on first use, kept
// until the process ends; default priority).
static int device_streams(DeviceStreams** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  std::lock_guard<std::mutex> lk(g_dsmu);
  if ((int)g_ds.size() <= dev) g_ds.resize(dev + 1, nullptr);
  if (!g_ds[dev]) {
    DeviceStreams* d = new DeviceStreams();
    for (int i = 0; i < kMaxGroups - 1; ++i) {
      if ((e = hipStreamCreateWithFlags(&d->s[i], hipStreamNonBlocking)) != hipSuccess) return (int)e;
      if ((e = hipEventCreateWithFlags(&d->join[i], hipEventDisableTiming)) != hipSuccess) return (int)e;
    }
    if ((e = hipEventCreateWithFlags(&d->fork, hipEventDisableTiming)) != hipSuccess) return (int)e;
    g_ds[dev] = d;
  }
  *out = g_ds[dev];
  return 0;
}

static int run_groups(GroupPlan& gp, char* ws, int prec_f32, const LaunchScalars& s, int steps, void* stream) {
  const int G = (int)gp.plans.size();
  if (G == 1) return run_plan(gp.plans[0], ws + gp.offs[0], prec_f32, s, steps, stream);
  DeviceStreams* d = nullptr;
  int r = device_streams(&d);
  if (r) return fail(DMUON_E_HIP, std::string("stream setup: ") + hip_error_string(r));
  std::lock_guard<std::mutex> lk(d->mu);
  hipStream_t caller = (hipStream_t)stream;
  if ((r = (int)hipEventRecord(d->fork, caller)) != 0) return fail(DMUON_E_HIP, std::string("fork: ") + hip_error_string(r));
  for (int g = 1; g < G; ++g)
    if ((r = (int)hipStreamWaitEvent(d->s[g - 1], d->fork, 0)) != 0)
      return fail(DMUON_E_HIP, std::string("fork wait: ") + hip_error_string(r));
  int rc = DMUON_OK;
  for (int g = 0; g < G && rc == DMUON_OK; ++g)
    rc = run_plan(gp.plans[g], ws + gp.offs[g], prec_f32, s, steps, g == 0 ? stream : (void*)d->s[g - 1]);
  // join every library stream back, also after a failed launch
  for (int g = 1; g < G; ++g) {
    if ((r = (int)hipEventRecord(d->join[g - 1], d->s[g - 1])) != 0 ||
        (r = (int)hipStreamWaitEvent(caller, d->join[g - 1], 0)) != 0)
      if (rc == DMUON_OK) rc = fail(DMUON_E_HIP, std::string("join: ") + hip_error_string(r));
  }
  return rc;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
struct Range {
  uintptr_t lo, hi;
  bool ro;
};

static int check_alias(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  // sweep: any writable range must not intersect any other range
  uintptr_t max_hi_any = 0, max_hi_w = 0;
  for (size_t i = 0; i < rs.size(); ++i) {
    const Range& r = rs[i];
    if (i > 0) {
      if (r.lo < max_hi_w) return fail(DMUON_E_ALIAS, "buffers overlap (a written buffer is shared)");
      if (!r.ro && r.lo < max_hi_any) return fail(DMUON_E_ALIAS, "buffers overlap (a written buffer is shared)");
    }
    max_hi_any = std::max(max_hi_any, r.hi);
    if (!r.ro) max_hi_w = std::max(max_hi_w, r.hi);
  }
  return DMUON_OK;
}

static bool finite(float x) { return std::isfinite(x); }

static int check_cfg(const dmuon_step_cfg* cfg) {
  if (!cfg) return fail(DMUON_E_NULL, "cfg is NULL");
  if (cfg->prec != DMUON_PREC_BF16_MFMA && cfg->prec != DMUON_PREC_F32)
    return fail(DMUON_E_DTYPE, "unknown precision code " + std::to_string(cfg->prec));
  if (cfg->ns_steps < 0 || cfg->ns_steps > kMaxSteps)
    return fail(DMUON_E_CFG, "ns_steps must be in [0, 64], got " + std::to_string(cfg->ns_steps));
  if (!finite(cfg->eps) || cfg->eps < 0.f) return fail(DMUON_E_CFG, "eps must be finite and >= 0");
  if (!finite(cfg->lr) || !finite(cfg->momentum) || !finite(cfg->weight_decay) || !finite(cfg->a) ||
      !finite(cfg->b) || !finite(cfg->c) || !finite(cfg->grad_scale))
    return fail(DMUON_E_CFG, "hyper-parameters must be finite");
  return DMUON_OK;
}

static int collect_items(const dmuon_tensor* t, int32_t n, std::vector<Item>& items, std::vector<Range>* rs) {
  if (n < 0) return fail(DMUON_E_SHAPE, "n_tensors < 0");
  if (n > 0 && !t) return fail(DMUON_E_NULL, "tensors is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_tensor& x = t[i];
    const std::string who = "tensor " + std::to_string(i) + ": ";
    if (x.ndim < 2) return fail(DMUON_E_NDIM, who + "Muon needs >= 2 dims (1-D parameters belong to an element-wise optimizer)");
    if (x.ndim > 3) return fail(DMUON_E_NDIM, who + "at most 3 dims (batch, rows, cols) are supported");
    for (int d = 0; d < x.ndim; ++d)
      if (x.shape[d] < 0) return fail(DMUON_E_SHAPE, who + "negative dim");
    if (x.grad_dtype != DMUON_F32 && x.grad_dtype != DMUON_BF16)
      return fail(DMUON_E_DTYPE, who + "grad_dtype must be DMUON_F32 or DMUON_BF16");
    const int64_t batch = x.ndim == 3 ? x.shape[0] : 1;
    const int64_t rows = x.shape[x.ndim - 2], cols = x.shape[x.ndim - 1];
    if (rows > 65536 || cols > 65536) return fail(DMUON_E_SHAPE, who + "rows and cols must be <= 65536");
    if (batch > (int64_t)1 << 30) return fail(DMUON_E_SHAPE, who + "batch too large");
    const int64_t numel = batch * rows * cols;
    if (numel == 0) continue;
    if (!x.grad || !x.momentum || !x.master) return fail(DMUON_E_NULL, who + "grad, momentum and master must be set");
    if (rs) {
      const size_t gs = x.grad_dtype == DMUON_BF16 ? 2 : 4;
      rs->push_back({(uintptr_t)x.grad, (uintptr_t)x.grad + numel * gs, true});
      rs->push_back({(uintptr_t)x.momentum, (uintptr_t)x.momentum + numel * 4, false});
      rs->push_back({(uintptr_t)x.master, (uintptr_t)x.master + numel * 4, false});
      if (x.ns_out) rs->push_back({(uintptr_t)x.ns_out, (uintptr_t)x.ns_out + numel * 4, false});
      if (x.param_out) rs->push_back({(uintptr_t)x.param_out, (uintptr_t)x.param_out + numel * 2, false});
    }
    items.push_back({batch, rows, cols, x.grad, x.grad_dtype == DMUON_BF16, x.momentum, x.master, x.ns_out,
                     x.param_out});
  }
  return DMUON_OK;
}

static int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return DMUON_OK;
  if (!ws) return fail(DMUON_E_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws & 255) return fail(DMUON_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(DMUON_E_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                       std::to_string(have));
  return DMUON_OK;
}

// The table copy reads a pinned staging buffer that later calls reuse: captured
// into a graph, its replays would read whatever that buffer then holds.
static int refuse_capture(void* stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
  if (e != hipSuccess) return fail(DMUON_E_HIP, std::string("stream query: ") + hip_error_string((int)e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(DMUON_E_HIP, "the stream is capturing a graph: the step stages its tables through a reused "
                             "host buffer and cannot be captured");
  return DMUON_OK;
}

static int test_fail_hook() {
  // DMUON_TEST_FAIL_AT=plan makes a valid call fail as a HIP error would, before
  // anything is enqueued (used by the host-side failure tests).
  const char* v = std::getenv("DMUON_TEST_FAIL_AT");
  if (v && std::strcmp(v, "plan") == 0) return fail(DMUON_E_HIP, "forced failure (DMUON_TEST_FAIL_AT=plan)");
  return DMUON_OK;
}

// ---- the adamw route ------------------------------------------------------
struct AdamwPlan {
  std::vector<AdamwProblem> probs;
  std::vector<int32_t> prefix;      // n + 1
  int64_t total_wg = 0;
  size_t off_prefix = 0, bytes = 0;
};

static int check_adamw_cfg(const dmuon_adamw_cfg* cfg) {
  if (!cfg) return fail(DMUON_E_NULL, "cfg is NULL");
  if (!finite(cfg->lr) || !finite(cfg->beta1) || !finite(cfg->beta2) || !finite(cfg->eps) ||
      !finite(cfg->weight_decay) || !finite(cfg->grad_scale))
    return fail(DMUON_E_CFG, "hyper-parameters must be finite");
  if (cfg->lr < 0.f) return fail(DMUON_E_CFG, "lr must be >= 0");
  if (cfg->beta1 < 0.f || cfg->beta1 >= 1.f || cfg->beta2 < 0.f || cfg->beta2 >= 1.f)
    return fail(DMUON_E_CFG, "beta1 and beta2 must be in [0, 1)");
  if (!(cfg->eps > 0.f)) return fail(DMUON_E_CFG, "eps must be > 0");
  if (cfg->step < 1) return fail(DMUON_E_CFG, "step counts from 1");
  return DMUON_OK;
}

static int collect_adamw(const dmuon_adamw_tensor* t, int32_t n, std::vector<const dmuon_adamw_tensor*>& items,
                         std::vector<Range>* rs) {
  if (n < 0) return fail(DMUON_E_SHAPE, "n_tensors < 0");
  if (n > 0 && !t) return fail(DMUON_E_NULL, "tensors is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const dmuon_adamw_tensor& x = t[i];
    const std::string who = "tensor " + std::to_string(i) + ": ";
    if (x.numel < 0) return fail(DMUON_E_SHAPE, who + "numel < 0");
    if (x.numel > ((int64_t)1 << 40)) return fail(DMUON_E_SHAPE, who + "numel too large");
    if (x.reserved != 0) return fail(DMUON_E_SHAPE, who + "reserved must be 0");
    if (x.grad_dtype != DMUON_F32 && x.grad_dtype != DMUON_BF16)
      return fail(DMUON_E_DTYPE, who + "grad_dtype must be DMUON_F32 or DMUON_BF16");
    if (x.numel == 0) continue;
    if (!x.grad || !x.param || !x.exp_avg || !x.exp_avg_sq)
      return fail(DMUON_E_NULL, who + "grad, param, exp_avg and exp_avg_sq must be set");
    if (rs) {
      const size_t gs = x.grad_dtype == DMUON_BF16 ? 2 : 4;
      const uintptr_t nb = (uintptr_t)x.numel;
      rs->push_back({(uintptr_t)x.grad, (uintptr_t)x.grad + nb * gs, true});
      rs->push_back({(uintptr_t)x.param, (uintptr_t)x.param + nb * 4, false});
      rs->push_back({(uintptr_t)x.exp_avg, (uintptr_t)x.exp_avg + nb * 4, false});
      rs->push_back({(uintptr_t)x.exp_avg_sq, (uintptr_t)x.exp_avg_sq + nb * 4, false});
      if (x.param_out) rs->push_back({(uintptr_t)x.param_out, (uintptr_t)x.param_out + nb * 2, false});
    }
    items.push_back(&x);
  }
  return DMUON_OK;
}

static int build_adamw_plan(const std::vector<const dmuon_adamw_tensor*>& items, AdamwPlan& pl) {
  const int n = (int)items.size();
  pl.probs.assign(n, AdamwProblem{});
  pl.prefix.assign(n + 1, 0);
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    const dmuon_adamw_tensor& x = *items[i];
    AdamwProblem& P = pl.probs[i];
    P.numel = x.numel;
    P.grad_bf16 = x.grad_dtype == DMUON_BF16;
    P.chunks = (int32_t)cdiv(x.numel, kElemChunk);
    P.wg0 = (int32_t)wg;
    P.grad = x.grad;
    P.param = x.param;
    P.m = x.exp_avg;
    P.v = x.exp_avg_sq;
    P.pub = x.param_out;
    pl.prefix[i] = (int32_t)wg;
    wg += P.chunks;
    if (wg > INT32_MAX) return fail(DMUON_E_SHAPE, "too many workgroups in one launch");
  }
  pl.prefix[n] = (int32_t)wg;
  pl.total_wg = wg;
  pl.off_prefix = align256((size_t)n * sizeof(AdamwProblem));
  pl.bytes = n ? align256(pl.off_prefix + (size_t)(n + 1) * sizeof(int32_t)) : 0;
  return DMUON_OK;
}

}  // namespace dmuon

using namespace dmuon;

extern "C" {

int32_t dmuon_abi_version(void) { return 3; }

const char* dmuon_last_error(void) { return g_err.c_str(); }

int dmuon_muon_step_workspace_size(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg,
                                   size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DMUON_E_NULL, "bytes is NULL");
  int e = check_cfg(cfg);
  if (e) return e;
  std::vector<Item> items;
  if ((e = collect_items(tensors, n, items, nullptr))) return e;
  if (items.empty()) {
    *bytes = 0;
    return DMUON_OK;
  }
  GroupPlan gp;
  if ((e = plan_groups(items, cfg->prec == DMUON_PREC_F32, nullptr, gp))) return e;
  *bytes = gp.bytes;
  return DMUON_OK;
}

int dmuon_muon_step(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_err.clear();
  int e = check_cfg(cfg);
  if (e) return e;
  std::vector<Item> items;
  std::vector<Range> rs;
  if ((e = collect_items(tensors, n, items, &rs))) return e;
  if (items.empty()) return DMUON_OK;
  if ((e = check_alias(rs))) return e;
  const int f32 = cfg->prec == DMUON_PREC_F32;
  GroupPlan gp;
  if ((e = plan_groups(items, f32, nullptr, gp))) return e;
  if ((e = check_workspace(workspace, workspace_bytes, gp.bytes))) return e;
  const uintptr_t wlo = (uintptr_t)workspace, whi = wlo + gp.bytes;
  for (const Range& r : rs)
    if (r.lo < whi && wlo < r.hi) return fail(DMUON_E_ALIAS, "workspace overlaps a tensor buffer");
  if ((e = test_fail_hook())) return e;
  if ((e = refuse_capture(stream))) return e;
  GroupPlan real;
  if ((e = plan_groups(items, f32, (char*)workspace, real))) return e;
  LaunchScalars s{};
  s.mu = cfg->momentum;
  s.lr = cfg->lr;
  s.decay = (float)(1.0 - (double)cfg->lr * (double)cfg->weight_decay);
  s.eps = cfg->eps;
  s.a = cfg->a;
  s.b = cfg->b;
  s.c = cfg->c;
  s.has_momentum = 1;
  s.normalize = 1;
  s.write_master = 1;
  s.gscale = cfg->grad_scale;
  return run_groups(real, (char*)workspace, f32, s, cfg->ns_steps, stream);
}

int dmuon_ns_batched_workspace_size(int64_t batch, int64_t rows, int64_t cols, int32_t prec, int32_t steps,
                                    size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DMUON_E_NULL, "bytes is NULL");
  if (prec != DMUON_PREC_BF16_MFMA && prec != DMUON_PREC_F32) return fail(DMUON_E_DTYPE, "unknown precision code");
  if (steps < 0 || steps > kMaxSteps) return fail(DMUON_E_CFG, "steps must be in [0, 64]");
  if (batch < 0 || rows < 0 || cols < 0) return fail(DMUON_E_SHAPE, "negative dim");
  if (rows > 65536 || cols > 65536 || batch > (int64_t)1 << 30) return fail(DMUON_E_SHAPE, "dim too large");
  if (batch * rows * cols == 0) {
    *bytes = 0;
    return DMUON_OK;
  }
  std::vector<Item> items{{batch, rows, cols, nullptr, 0, nullptr, nullptr, nullptr, nullptr}};
  Plan pl;
  int e = build_plan(items, prec == DMUON_PREC_F32, pl, nullptr);
  if (e) return e;
  *bytes = pl.bytes;
  return DMUON_OK;
}

int dmuon_ns_batched(const void* x, int32_t x_dtype, float* out, int64_t batch, int64_t rows, int64_t cols, float a,
                     float b, float c, int32_t steps, float eps, int32_t normalize, int32_t prec, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (prec != DMUON_PREC_BF16_MFMA && prec != DMUON_PREC_F32) return fail(DMUON_E_DTYPE, "unknown precision code");
  if (x_dtype != DMUON_F32 && x_dtype != DMUON_BF16) return fail(DMUON_E_DTYPE, "x_dtype must be DMUON_F32 or DMUON_BF16");
  if (steps < 0 || steps > kMaxSteps) return fail(DMUON_E_CFG, "steps must be in [0, 64]");
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
    return fail(DMUON_E_CFG, "a, b, c, eps must be finite and eps >= 0");
  if (normalize != 0 && normalize != 1) return fail(DMUON_E_CFG, "normalize must be 0 or 1");
  if (batch < 0 || rows < 0 || cols < 0) return fail(DMUON_E_SHAPE, "negative dim");
  if (rows > 65536 || cols > 65536 || batch > (int64_t)1 << 30) return fail(DMUON_E_SHAPE, "dim too large");
  const int64_t numel = batch * rows * cols;
  if (numel == 0) return DMUON_OK;
  if (!x || !out) return fail(DMUON_E_NULL, "x and out must be set");
  const size_t xs = x_dtype == DMUON_BF16 ? 2 : 4;
  std::vector<Range> rs{{(uintptr_t)x, (uintptr_t)x + numel * xs, true},
                        {(uintptr_t)out, (uintptr_t)out + numel * 4, false}};
  int e = check_alias(rs);
  if (e) return e;
  std::vector<Item> items{{batch, rows, cols, x, x_dtype == DMUON_BF16, nullptr, nullptr, out, nullptr}};
  const int f32 = prec == DMUON_PREC_F32;
  Plan pl;
  if ((e = build_plan(items, f32, pl, nullptr))) return e;
  if ((e = check_workspace(workspace, workspace_bytes, pl.bytes))) return e;
  const uintptr_t wlo = (uintptr_t)workspace, whi = wlo + pl.bytes;
  for (const Range& r : rs)
    if (r.lo < whi && wlo < r.hi) return fail(DMUON_E_ALIAS, "workspace overlaps x or out");
  if ((e = test_fail_hook())) return e;
  if ((e = refuse_capture(stream))) return e;
  Plan real;
  if ((e = build_plan(items, f32, real, (char*)workspace))) return e;
  LaunchScalars s{};
  s.eps = eps;
  s.a = a;
  s.b = b;
  s.c = c;
  s.has_momentum = 0;
  s.normalize = normalize;
  s.write_master = 0;
  s.gscale = 1.f;
  return run_plan(real, (char*)workspace, f32, s, steps, stream);
}

int dmuon_adamw_step_workspace_size(const dmuon_adamw_tensor* tensors, int32_t n, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(DMUON_E_NULL, "bytes is NULL");
  std::vector<const dmuon_adamw_tensor*> items;
  int e = collect_adamw(tensors, n, items, nullptr);
  if (e) return e;
  AdamwPlan pl;
  if ((e = build_adamw_plan(items, pl))) return e;
  *bytes = pl.bytes;
  return DMUON_OK;
}

int dmuon_adamw_step(const dmuon_adamw_tensor* tensors, int32_t n, const dmuon_adamw_cfg* cfg, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  int e = check_adamw_cfg(cfg);
  if (e) return e;
  std::vector<const dmuon_adamw_tensor*> items;
  std::vector<Range> rs;
  if ((e = collect_adamw(tensors, n, items, &rs))) return e;
  if (items.empty()) return DMUON_OK;
  if ((e = check_alias(rs))) return e;
  AdamwPlan pl;
  if ((e = build_adamw_plan(items, pl))) return e;
  if ((e = check_workspace(workspace, workspace_bytes, pl.bytes))) return e;
  const uintptr_t wlo = (uintptr_t)workspace, whi = wlo + pl.bytes;
  for (const Range& r : rs)
    if (r.lo < whi && wlo < r.hi) return fail(DMUON_E_ALIAS, "workspace overlaps a tensor buffer");
  if ((e = test_fail_hook())) return e;
  if ((e = refuse_capture(stream))) return e;
  std::vector<char> host(pl.bytes, 0);
  std::memcpy(host.data(), pl.probs.data(), pl.probs.size() * sizeof(AdamwProblem));
  std::memcpy(host.data() + pl.off_prefix, pl.prefix.data(), pl.prefix.size() * sizeof(int32_t));
  char* ws = (char*)workspace;
  e = stage_upload(ws, host.data(), host.size(), stream);
  if (e) return fail(DMUON_E_HIP, std::string("table upload: ") + hip_error_string(e));
  // bias corrections in double on the host (step is exact as an integer)
  const double b1 = cfg->beta1, b2 = cfg->beta2;
  const double bc1 = 1.0 - std::pow(b1, (double)cfg->step);
  const double bc2 = 1.0 - std::pow(b2, (double)cfg->step);
  AdamwScalars s{};
  s.decay = (float)(1.0 - (double)cfg->lr * (double)cfg->weight_decay);
  s.step_size = (float)((double)cfg->lr / bc1);
  s.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  s.eps = cfg->eps;
  s.beta1 = cfg->beta1;
  s.one_m_beta1 = (float)(1.0 - b1);
  s.beta2 = cfg->beta2;
  s.one_m_beta2 = (float)(1.0 - b2);
  s.gscale = cfg->grad_scale;
  AdamwTable tab;
  tab.probs = (const AdamwProblem*)ws;
  tab.wg_prefix = (const int32_t*)(ws + pl.off_prefix);
  tab.n_probs = (int32_t)pl.probs.size();
  tab.total_wg = (int32_t)pl.total_wg;
  const int r = launch_adamw(tab, s, stream);
  if (r) return fail(DMUON_E_HIP, std::string("launch failed: ") + hip_error_string(r));
  return DMUON_OK;
}

int dmuon_gemm_nt(const void* A, const void* B, float* C, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                  int64_t ldc, int32_t dtype, void* stream) {
  g_err.clear();
  if (dtype != DMUON_F32 && dtype != DMUON_BF16) return fail(DMUON_E_DTYPE, "dtype must be DMUON_F32 or DMUON_BF16");
  if (M < 0 || N < 0 || K < 0) return fail(DMUON_E_SHAPE, "negative dim");
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return fail(DMUON_E_SHAPE, "dim too large");
  if (M == 0 || N == 0) return DMUON_OK;
  if (!A || !B || !C) return fail(DMUON_E_NULL, "A, B and C must be set");
  const int64_t kpad = round_up(K, kLdAlign);
  if (lda % kLdAlign || ldb % kLdAlign || lda < kpad || ldb < kpad || ldc < N)
    return fail(DMUON_E_SHAPE, "lda, ldb must be multiples of 64 and >= round_up(K, 64); ldc >= N");
  if (((uintptr_t)A & 15) || ((uintptr_t)B & 15)) return fail(DMUON_E_SHAPE, "A and B must be 16-byte aligned");
  if (K == 0) {
    // the kernel still runs one K tile of (required zero) padding
  }
  const int r = launch_gemm_nt(A, B, C, M, N, K == 0 ? 1 : K, lda, ldb, ldc, dtype == DMUON_F32, stream);
  if (r) return fail(DMUON_E_HIP, std::string("launch failed: ") + hip_error_string(r));
  return DMUON_OK;
}

int dmuon_phase_timing(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return DMUON_OK;
}

int dmuon_phase_timing_read(double* ms, int64_t* count, int32_t n) {
  g_err.clear();
  if ((!ms || !count) && n > 0) return fail(DMUON_E_NULL, "ms and count must be set");
  std::lock_guard<std::mutex> lk(g_tmu);
  for (int i = 0; i < n; ++i) {
    ms[i] = 0.0;
    count[i] = 0;
  }
  int rc = DMUON_OK;
  for (TimedLaunch& tl : g_timed) {
    if (hipEventSynchronize(tl.b) != hipSuccess) rc = fail(DMUON_E_HIP, "event synchronize failed");
    float t = 0.f;
    if (rc == DMUON_OK && hipEventElapsedTime(&t, tl.a, tl.b) == hipSuccess && tl.phase < n) {
      ms[tl.phase] += t;
      count[tl.phase] += 1;
    }
    g_evpool.push_back(tl.a);
    g_evpool.push_back(tl.b);
  }
  g_timed.clear();
  return rc;
}

}  // extern "C"
