// C entry points of libdmuon_ns: validation, planning, launch sequence, timing.
//
// The step follows the DMuon "架构设计" (Architecture design) page: §1 gives the
// Newton–Schulz equation, §2 says only the owner runs NS + momentum + weight
// decay + parameter update on its local full-precision copy without any
// communication; the HSDP guide ("what happens underneath", step 3) repeats it.
// Rank checks follow the MindSpore parameter-grouping page §2.1 / §4.1 (fewer
// than two dims is an error) and §2.2 / §6 (the matrix is the last two dims).
#include <hip/hip_runtime_api.h>

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
// tables
//
// A call's tables (problem descriptors and per-phase workgroup prefixes) are
// built on the host and carried into the workspace in the kernel arguments of
// small copy kernels on the caller's stream (launch_write_table), so the
// library keeps no host staging memory, no host buffer has to outlive the
// call, and a captured graph replays the same bytes.  Every problem entry
// carries a tag, the FNV-1a hash of the whole host table; the step's kernels
// are launched with the tag they expect, and a workgroup that finds another
// one exits before touching memory, so a launch on a workspace that does not
// hold its plan's table does nothing.
// ---------------------------------------------------------------------------
static uint32_t fnv1a(const char* p, size_t n) {
  uint32_t h = 2166136261u;
  for (size_t i = 0; i < n; ++i) {
    h ^= (uint8_t)p[i];
    h *= 16777619u;
  }
  return h;
}

// Per-call debugging switches, read from the environment once per call.
//
// DMUON_TEST_FAIL_AT (failure-handling tests) names the point at which a valid
// call returns DMUON_E_HIP as a failed HIP call would: "plan" (after
// validation, before anything is enqueued), "table" (the table copy), or a
// phase name (that phase's first launch; earlier launches are enqueued).
//
// DMUON_DEBUG_SYNC (set and not "0") waits for every launch to finish before
// the next is enqueued and returns DMUON_E_HIP naming the launch whose wait
// reported an error, so an asynchronous fault is tied to its phase.  The wait
// is skipped on a stream under graph capture, where it is not allowed.
static const char* const kPhaseNames[PH_COUNT] = {"ingest", "norm",   "gram",    "square",
                                                  "apply",  "update", "gemm_nt", "adamw"};
struct CallEnv {
  int where = -3;     // -3 none, -2 plan, -1 table, else a phase id
  bool sync = false;  // DMUON_DEBUG_SYNC
};
static CallEnv call_env() {
  CallEnv f;
  const char* d = std::getenv("DMUON_DEBUG_SYNC");
  f.sync = d && *d && std::strcmp(d, "0") != 0;
  const char* v = std::getenv("DMUON_TEST_FAIL_AT");
  if (!v) return f;
  if (std::strcmp(v, "plan") == 0) f.where = -2;
  else if (std::strcmp(v, "table") == 0) f.where = -1;
  for (int i = 0; i < PH_COUNT; ++i)
    if (std::strcmp(v, kPhaseNames[i]) == 0) f.where = i;
  return f;
}
static int forced(const CallEnv& f, int where) {
  if (f.where != where) return DMUON_OK;
  return fail(DMUON_E_HIP, std::string("forced failure (DMUON_TEST_FAIL_AT=") + std::getenv("DMUON_TEST_FAIL_AT") + ")");
}
static int settle(const CallEnv& f, void* stream, const char* what) {
  if (!f.sync) return DMUON_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  int r = (int)hipStreamIsCapturing((hipStream_t)stream, &cs);
  if (r == 0 && cs != hipStreamCaptureStatusNone) return DMUON_OK;
  if (r == 0) r = (int)hipStreamSynchronize((hipStream_t)stream);
  if (r) return fail(DMUON_E_HIP, std::string(what) + " (DMUON_DEBUG_SYNC): " + hip_error_string(r));
  return DMUON_OK;
}

static int write_table(void* dst, const std::vector<char>& host, void* stream, const CallEnv& fa) {
  int e = forced(fa, -1);
  if (e) return e;
  e = launch_write_table(dst, host.data(), host.size(), stream);
  if (e) return fail(DMUON_E_HIP, std::string("table copy: ") + hip_error_string(e));
  return settle(fa, stream, "table");
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
  uint32_t tag = 0;
};

// The device image of the plan's tables, with every entry's tag set.
static std::vector<char> seal(Plan& pl) {
  std::vector<char> host(pl.table_bytes, 0);
  for (DevProblem& P : pl.probs) P.tag = 0;
  auto fill = [&] {
    std::memcpy(host.data(), pl.probs.data(), pl.probs.size() * sizeof(DevProblem));
    std::memcpy(host.data() + pl.off_prefix, pl.prefix.data(), pl.prefix.size() * sizeof(int32_t));
  };
  fill();
  pl.tag = fnv1a(host.data(), host.size());
  for (DevProblem& P : pl.probs) P.tag = pl.tag;
  fill();
  return host;
}

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
    // the iterate: fp32 on the fp32 path; on the bf16 path its part below the
    // bf16 operand copy, one signed byte per value plus one exponent byte per 16
    P.xf = (float*)carve((size_t)(b * P.apply_tr * P.apply_tc) * kTile * kTile / 16 * (prec_f32 ? 64 : 17));
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

// Enqueue the phases of one plan whose tables are in the workspace at ws.
static int launch_plan(const Plan& pl, char* ws, int prec_f32, const LaunchScalars& base_s, int steps,
                       void* stream, const CallEnv& fa) {
  LaunchTable tab;
  tab.probs = (const DevProblem*)ws;
  tab.wg_prefix = (const int32_t*)(ws + pl.off_prefix);
  tab.scal = (float*)(ws + pl.off_scal);
  tab.n_probs = (int32_t)pl.probs.size();
  tab.tag = pl.tag;
  auto go = [&](int ph, const LaunchScalars& s) -> int {
    int e = forced(fa, ph);
    if (e) return e;
    tab.total_wg = (int32_t)pl.total_wg[ph];
    const int r = launch_phase(ph, prec_f32, tab, s, stream);
    if (r) return fail(DMUON_E_HIP, std::string("launch failed: ") + hip_error_string(r));
    return settle(fa, stream, kPhaseNames[ph]);
  };
  int e;
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
// launch sequence; group 0 runs on the caller's stream and the others on the
// side streams the caller passes, forked from it and joined back with events,
// so one group's tail rounds overlap another group's next phase.  Each slice's arithmetic is
// the same whatever its group, so results do not depend on the split.
// ---------------------------------------------------------------------------
constexpr int kMaxGroups = 4;

// Group count from the length of the apply phase on the 256 CUs of an MI355X,
// in rounds of 32-wide K stages (Σ tiles · stages / 256; a fixed count keeps the
// workspace size a host-only computation).  Measured, ms per step with
// 1 / 2 / 3 / 4 groups on caller-owned side streams:
// * short phases (under 1024 stage-rounds): four groups, whose tail rounds,
//   epilogues and launch gaps overlap each other's contractions (one d = 2048
//   layer, 196 stage-rounds: 2.51 / 2.34 / 2.36 / 2.31; 384 matrices of 512² and
//   256×1024, 80 stage-rounds: 2.50 / 2.27 / 2.26 / 2.26);
// * otherwise one: the tails are a small share, and one launch sequence keeps
//   the operand panels of neighbouring tiles together in each XCD's L2 (Llama
//   d = 4096 share, 6304 stage-rounds: 58.2 / 60.2; MLP/MoE mix, 14864:
//   116.1 / 122.0).
constexpr int kCusAssumed = 256;

// requested: the cfg's stream_groups (0: the rule above).
static int group_count(const std::vector<Item>& items, int requested) {
  double stages = 0;
  for (const Item& it : items)
    stages += (double)it.batch * cdiv(it.rows, kTile) * cdiv(it.cols, kTile) * cdiv(std::min(it.rows, it.cols), 32);
  const int g = requested >= 1 ? requested : (stages < 1024.0 * kCusAssumed ? 4 : 1);
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

// Split the items into G groups, size (base == nullptr) or lay out every group's plan.
static int plan_groups(const std::vector<Item>& items, int prec_f32, int requested, char* base, GroupPlan& gp) {
  const int G = group_count(items, requested);
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

// Copy every group's tables into the workspace, on the caller's stream.
static int write_groups(GroupPlan& gp, char* ws, void* stream, const CallEnv& fa) {
  for (size_t g = 0; g < gp.plans.size(); ++g) {
    const std::vector<char> host = seal(gp.plans[g]);
    const int e = write_table(ws + gp.offs[g], host, stream, fa);
    if (e) return e;
  }
  return DMUON_OK;
}

// Enqueue every group's phases.  Group 0 runs on `stream`, group g ≥ 1 on
// side[(g − 1) % n_side] (on `stream` too when n_side is 0).  The side streams
// fork from `stream` and join back to it through events made for this call and
// released before it returns (HIP keeps a recorded event's pending work alive).
static int launch_groups(GroupPlan& gp, char* ws, int prec_f32, const LaunchScalars& s, int steps, void* stream,
                         void* const* side, int n_side, const CallEnv& fa) {
  const int G = (int)gp.plans.size();
  for (Plan& pl : gp.plans) (void)seal(pl);       // the tags the kernels expect
  const int used = n_side > 0 ? std::min(G - 1, n_side) : 0;
  hipStream_t caller = (hipStream_t)stream;
  int r;
  if (used > 0) {
    hipEvent_t fork = nullptr;
    if ((r = (int)hipEventCreateWithFlags(&fork, hipEventDisableTiming)) != 0)
      return fail(DMUON_E_HIP, std::string("fork event: ") + hip_error_string(r));
    r = (int)hipEventRecord(fork, caller);
    for (int i = 0; i < used && r == 0; ++i) r = (int)hipStreamWaitEvent((hipStream_t)side[i], fork, 0);
    (void)hipEventDestroy(fork);
    if (r) return fail(DMUON_E_HIP, std::string("fork: ") + hip_error_string(r));
  }
  int rc = DMUON_OK;
  for (int g = 0; g < G && rc == DMUON_OK; ++g) {
    void* st = (g == 0 || used == 0) ? stream : side[(g - 1) % used];
    rc = launch_plan(gp.plans[g], ws + gp.offs[g], prec_f32, s, steps, st, fa);
  }
  // join every side stream back, also after a failed launch
  for (int i = 0; i < used; ++i) {
    hipEvent_t join = nullptr;
    r = (int)hipEventCreateWithFlags(&join, hipEventDisableTiming);
    if (r == 0) r = (int)hipEventRecord(join, (hipStream_t)side[i]);
    if (r == 0) r = (int)hipStreamWaitEvent(caller, join, 0);
    if (join) (void)hipEventDestroy(join);
    if (r && rc == DMUON_OK) rc = fail(DMUON_E_HIP, std::string("join: ") + hip_error_string(r));
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
  if (cfg->stream_groups < 0 || cfg->stream_groups > kMaxGroups)
    return fail(DMUON_E_CFG, "stream_groups must be in [0, 4], got " + std::to_string(cfg->stream_groups));
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

static int check_side(void* const* side, int32_t n_side) {
  if (n_side < 0) return fail(DMUON_E_CFG, "n_side_streams < 0");
  if (n_side > 0 && !side) return fail(DMUON_E_NULL, "side_streams is NULL");
  for (int32_t i = 0; i < n_side; ++i)
    if (!side[i]) return fail(DMUON_E_NULL, "side_streams[" + std::to_string(i) + "] is NULL (the null stream)");
  return DMUON_OK;
}

// Validation shared by the step entry points: cfg, tensors, overlaps, the
// workspace; on success `gp` holds the plan laid out on the workspace.
static int prepare_step(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                        size_t workspace_bytes, std::vector<Item>& items, GroupPlan& gp) {
  int e = check_cfg(cfg);
  if (e) return e;
  std::vector<Range> rs;
  if ((e = collect_items(tensors, n, items, &rs))) return e;
  if (items.empty()) return DMUON_OK;
  if ((e = check_alias(rs))) return e;
  const int f32 = cfg->prec == DMUON_PREC_F32;
  GroupPlan sized;
  if ((e = plan_groups(items, f32, cfg->stream_groups, nullptr, sized))) return e;
  if ((e = check_workspace(workspace, workspace_bytes, sized.bytes))) return e;
  const uintptr_t wlo = (uintptr_t)workspace, whi = wlo + sized.bytes;
  for (const Range& r : rs)
    if (r.lo < whi && wlo < r.hi) return fail(DMUON_E_ALIAS, "workspace overlaps a tensor buffer");
  return plan_groups(items, f32, cfg->stream_groups, (char*)workspace, gp);
}

static LaunchScalars step_scalars(const dmuon_step_cfg* cfg) {
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
  return s;
}

// ---- the adamw route ------------------------------------------------------
struct AdamwPlan {
  std::vector<AdamwProblem> probs;
  std::vector<int32_t> prefix;      // n + 1
  int64_t total_wg = 0;
  size_t off_prefix = 0, bytes = 0;
  uint32_t tag = 0;
};

static std::vector<char> seal(AdamwPlan& pl) {
  std::vector<char> host(pl.bytes, 0);
  for (AdamwProblem& P : pl.probs) P.tag = 0;
  auto fill = [&] {
    std::memcpy(host.data(), pl.probs.data(), pl.probs.size() * sizeof(AdamwProblem));
    std::memcpy(host.data() + pl.off_prefix, pl.prefix.data(), pl.prefix.size() * sizeof(int32_t));
  };
  fill();
  pl.tag = fnv1a(host.data(), host.size());
  for (AdamwProblem& P : pl.probs) P.tag = pl.tag;
  fill();
  return host;
}

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

int32_t dmuon_abi_version(void) { return 5; }

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
  if ((e = plan_groups(items, cfg->prec == DMUON_PREC_F32, cfg->stream_groups, nullptr, gp))) return e;
  *bytes = gp.bytes;
  return DMUON_OK;
}

int dmuon_muon_step_groups(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, int32_t* groups) {
  g_err.clear();
  if (!groups) return fail(DMUON_E_NULL, "groups is NULL");
  int e = check_cfg(cfg);
  if (e) return e;
  std::vector<Item> items;
  if ((e = collect_items(tensors, n, items, nullptr))) return e;
  *groups = items.empty() ? 0 : group_count(items, cfg->stream_groups);
  return DMUON_OK;
}

int dmuon_muon_step_prepare(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_err.clear();
  std::vector<Item> items;
  GroupPlan gp;
  int e = prepare_step(tensors, n, cfg, workspace, workspace_bytes, items, gp);
  if (e || items.empty()) return e;
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  return write_groups(gp, (char*)workspace, stream, fa);
}

int dmuon_muon_step_run(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* side_streams, int32_t n_side_streams) {
  g_err.clear();
  int e = check_side(side_streams, n_side_streams);
  if (e) return e;
  std::vector<Item> items;
  GroupPlan gp;
  if ((e = prepare_step(tensors, n, cfg, workspace, workspace_bytes, items, gp)) || items.empty()) return e;
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  return launch_groups(gp, (char*)workspace, cfg->prec == DMUON_PREC_F32, step_scalars(cfg), cfg->ns_steps,
                       stream, side_streams, n_side_streams, fa);
}

int dmuon_muon_step(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                    size_t workspace_bytes, void* stream, void* const* side_streams, int32_t n_side_streams) {
  g_err.clear();
  int e = check_side(side_streams, n_side_streams);
  if (e) return e;
  std::vector<Item> items;
  GroupPlan gp;
  if ((e = prepare_step(tensors, n, cfg, workspace, workspace_bytes, items, gp)) || items.empty()) return e;
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  if ((e = write_groups(gp, (char*)workspace, stream, fa))) return e;
  return launch_groups(gp, (char*)workspace, cfg->prec == DMUON_PREC_F32, step_scalars(cfg), cfg->ns_steps,
                       stream, side_streams, n_side_streams, fa);
}

int dmuon_debug_slice_buffers(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* workspace,
                              size_t workspace_bytes, int32_t tensor, int64_t slice, dmuon_debug_slice* out) {
  g_err.clear();
  if (!out) return fail(DMUON_E_NULL, "out is NULL");
  std::vector<Item> items;
  GroupPlan gp;
  int e = prepare_step(tensors, n, cfg, workspace, workspace_bytes, items, gp);
  if (e) return e;
  if (tensor < 0 || tensor >= n) return fail(DMUON_E_SHAPE, "tensor index out of range");
  const dmuon_tensor& t = tensors[tensor];
  const int64_t batch = t.ndim == 3 ? t.shape[0] : 1;
  if (slice < 0 || slice >= batch) return fail(DMUON_E_SHAPE, "slice index out of range");
  const bool f32 = cfg->prec == DMUON_PREC_F32;
  const size_t esz = f32 ? 4 : 2;
  // the momentum buffer is written, so no two tensors share it: it names the problem
  for (size_t g = 0; g < gp.plans.size(); ++g) {
    const Plan& pl = gp.plans[g];
    for (const DevProblem& P : pl.probs) {
      if (P.mom != t.momentum) continue;
      dmuon_debug_slice d{};
      const int64_t ld_s = P.wide ? P.ld_n : P.ld_m;
      if (f32) {
        d.x_copy = (const char*)P.xg + (size_t)(slice * P.m * P.ld_n) * esz;
        d.x_rows = P.m;
        d.x_ld = P.ld_n;
        d.x_oriented = 1;
      } else {
        d.x_copy = (const char*)P.xs[0] + (size_t)(slice * P.rows * ld_s) * esz;
        d.x_rows = P.rows;
        d.x_ld = ld_s;
        d.x_oriented = 0;
      }
      d.elem_bytes = (int32_t)esz;
      d.a_prime = (const char*)P.ap + (size_t)(slice * P.m * P.ld_m) * esz;
      d.b_prime = (const char*)P.bp + (size_t)(slice * P.m * P.ld_m) * esz;
      d.ld_m = P.ld_m;
      d.scalars = (const float*)((char*)workspace + gp.offs[g] + pl.off_scal) + (P.slice_base + slice) * kScalStride;
      d.m = P.m;
      d.n = P.n;
      d.wide = P.wide;
      *out = d;
      return DMUON_OK;
    }
  }
  return fail(DMUON_E_SHAPE, "the tensor has no slices (a zero-size dim)");
}

int dmuon_muon_step_noalloc(const dmuon_tensor* tensors, int32_t n, const dmuon_step_cfg* cfg, void* stream) {
  g_err.clear();
  int e = check_cfg(cfg);
  if (e) return e;
  if (cfg->stream_groups > 1) return fail(DMUON_E_CFG, "the allocation-free step runs as one group: stream_groups must be 0 or 1");
  std::vector<Item> items;
  std::vector<Range> rs;
  if ((e = collect_items(tensors, n, items, &rs))) return e;
  if (items.empty()) return DMUON_OK;
  if ((e = check_alias(rs))) return e;
  const int f32 = cfg->prec == DMUON_PREC_F32;
  GroupPlan sized;
  if ((e = plan_groups(items, f32, 1, nullptr, sized))) return e;
  if (sized.bytes > kScratchBytes)
    return fail(DMUON_E_WORKSPACE, "the allocation-free step needs " + std::to_string(sized.bytes) +
                                       " bytes of scratch; the library's static scratch holds " +
                                       std::to_string(kScratchBytes));
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  void* scr = nullptr;
  const int r = scratch_region(&scr);
  if (r) return fail(DMUON_E_HIP, std::string("scratch lookup: ") + hip_error_string(r));
  GroupPlan gp;
  if ((e = plan_groups(items, f32, 1, (char*)scr, gp))) return e;
  if ((e = write_groups(gp, (char*)scr, stream, fa))) return e;
  return launch_groups(gp, (char*)scr, f32, step_scalars(cfg), cfg->ns_steps, stream, nullptr, 0, fa);
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
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  Plan real;
  if ((e = build_plan(items, f32, real, (char*)workspace))) return e;
  if ((e = write_table(workspace, seal(real), stream, fa))) return e;
  LaunchScalars s{};
  s.eps = eps;
  s.a = a;
  s.b = b;
  s.c = c;
  s.has_momentum = 0;
  s.normalize = normalize;
  s.write_master = 0;
  s.gscale = 1.f;
  return launch_plan(real, (char*)workspace, f32, s, steps, stream, fa);
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
  const CallEnv fa = call_env();
  if ((e = forced(fa, -2))) return e;
  char* ws = (char*)workspace;
  if ((e = write_table(ws, seal(pl), stream, fa))) return e;
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
  tab.tag = pl.tag;
  if ((e = forced(fa, PH_ADAMW))) return e;
  const int r = launch_adamw(tab, s, stream);
  if (r) return fail(DMUON_E_HIP, std::string("launch failed: ") + hip_error_string(r));
  return settle(fa, stream, "adamw");
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
  return settle(call_env(), stream, "gemm_nt");
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
