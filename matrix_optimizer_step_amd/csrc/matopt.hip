// Host side of libmatopt: the C ABI declared in include/matopt.h.
//
// Each entry point validates its arguments synchronously, looks up (or builds
// once) a plan for its list of shapes -- descriptor templates plus the tile
// and task tables of every launch, in one device buffer the library owns --
// binds this call's pointers into the descriptors (bind_kernel: the pointers
// travel as kernel arguments), and enqueues the whole step on the caller's
// stream as a fixed sequence of grouped launches (every launch covers every
// matrix of the batch):
//
//   muon_step_batched        bind -> prep (momentum, norm partials, X0) ->
//                            finalize -> ns_steps x {Gram, polynomial, apply}
//                            (the last apply folds the update into W) |
//                            scale_out if ns_steps == 0
//   ns_orthogonalize_batched same with no momentum; the last apply writes O
//   rmnp_step_batched        bind -> one fused row kernel launch per width class
//
// A plan depends on the shapes only, so a caller whose tensors move between
// calls (gradients reallocated every step) reuses it: after the first call
// with a list of shapes nothing is allocated, copied from the host or
// synchronised.  Descriptors of the Newton-Schulz calls live in the caller's
// workspace; those of the calls without a workspace in a slot of the plan,
// which is why the calls that use one plan are chained across streams.
//
// Tile tables are ordered longest-K first (largest work first, the greedy the
// MatrixFSDP owner planner uses for roles, section 4.1, Algorithm 1), so that
// the tail of each launch is made of short tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/matopt.h"
#include "common.hpp"
#include "tile_schedule.hpp"

using namespace matopt;

namespace {

thread_local std::string g_detail;

matopt_status fail(matopt_status s, const std::string& msg) {
  g_detail = msg;
  return s;
}

// ---------------------------------------------------------------- device check
std::mutex g_dev_mu;
std::map<int, bool> g_dev_ok;

matopt_status check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MATOPT_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev_ok.find(dev);
  if (it == g_dev_ok.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(MATOPT_ERR_DEVICE, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = g_dev_ok.emplace(dev, ok).first;
    if (!ok) g_detail = std::string("device arch ") + prop.gcnArchName + " is not gfx950";
  }
  if (!it->second) return fail(MATOPT_ERR_DEVICE, "current device is not gfx950 (MI355X)");
  *dev_out = dev;
  return MATOPT_OK;
}

// ---------------------------------------------------------------- geometry
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// Compute modes of the Newton-Schulz entry points beyond the storage dtypes:
// bf16 storage with the split-precision iterate (MATOPT_BF16_SPLIT).
constexpr int DT_BF16_SPLIT = 2;
int sdt(int dt) { return dt == DT_BF16_SPLIT ? DT_BF16 : dt; }   // storage dtype
int esize(int dt) { return sdt(dt) == DT_BF16 ? 2 : 4; }
int gemm_tile(int dt) { return sdt(dt) == DT_BF16 ? kTileBf16 : kTileF32; }

struct Geo {
  int64_t rows, cols;
  int m, n, mp, np;
  bool transposed;
  int prep_tr, prep_tc;
};

Geo geometry(int64_t rows, int64_t cols, int dt) {
  Geo g;
  g.rows = rows;
  g.cols = cols;
  g.transposed = rows > cols;
  g.m = (int)(g.transposed ? cols : rows);
  g.n = (int)(g.transposed ? rows : cols);
  const int t = gemm_tile(dt);
  g.mp = (int)round_up(g.m, t);
  g.np = (int)round_up(g.n, t);
  const int rows_p = g.transposed ? g.np : g.mp;
  const int cols_p = g.transposed ? g.mp : g.np;
  g.prep_tr = rows_p / kPrepTile;
  g.prep_tc = cols_p / (g.transposed && sdt(dt) == DT_BF16 ? kPrepTileT : kPrepTile);
  return g;
}

struct Layout {
  std::vector<size_t> x0, x1, a, b;
  size_t partials = 0, xs = 0, desc = 0, total = 0;
  int n_prep = 0;
  std::vector<int> prep_off;
};

constexpr int64_t kMaxSide = 1 << 20;
constexpr int64_t kMaxElems = int64_t(1) << 32;

Layout layout(const std::vector<Geo>& geo, int dt) {
  Layout L;
  const size_t es = esize(dt);
  size_t off = 0;
  // split precision: each iterate buffer holds the bf16 high part over the low part
  const size_t xparts = dt == DT_BF16_SPLIT ? 2 : 1;
  for (const Geo& g : geo) {
    const size_t xb = align256((size_t)g.mp * g.np * es * xparts);
    const size_t ab = align256((size_t)g.mp * g.mp * es);
    L.x0.push_back(off); off += xb;
    L.x1.push_back(off); off += xb;
    L.a.push_back(off); off += ab;
    L.b.push_back(off); off += ab;
    L.prep_off.push_back(L.n_prep);
    L.n_prep += g.prep_tr * g.prep_tc;
  }
  L.partials = off;
  off += align256((size_t)L.n_prep * 4);
  L.xs = off;
  off += align256(geo.size() * 4);
  L.desc = off;   // this call's descriptors (written by bind_kernel)
  off += align256(geo.size() * sizeof(MatDesc));
  L.total = off;
  return L;
}

// ---------------------------------------------------------------- validation
bool finite(float x) { return std::isfinite(x); }

matopt_status check_shape(int64_t rows, int64_t cols, int i) {
  if (rows < 1 || cols < 1 || rows > kMaxSide || cols > kMaxSide || rows * cols > kMaxElems)
    return fail(MATOPT_ERR_SHAPE, "matrix " + std::to_string(i) + ": invalid shape " +
                                      std::to_string(rows) + "x" + std::to_string(cols));
  return MATOPT_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

struct Span {
  uintptr_t lo, hi;
  std::string what;
};

matopt_status check_overlap(std::vector<Span>& spans) {
  std::sort(spans.begin(), spans.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].lo < spans[i - 1].hi)
      return fail(MATOPT_ERR_ALIAS, spans[i - 1].what + " overlaps " + spans[i].what);
  return MATOPT_OK;
}

// ---------------------------------------------------------------- profiling
std::atomic<bool> g_prof{false};
std::mutex g_prof_mu;
struct ProfRec {
  int cls;
  hipEvent_t a, b;
};
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_ev_free;
double g_prof_ms[MATOPT_PROFILE_CLASSES];
int64_t g_prof_n[MATOPT_PROFILE_CLASSES];

hipEvent_t take_event() {
  if (!g_ev_free.empty()) {
    hipEvent_t e = g_ev_free.back();
    g_ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Clock counters of the bf16 GEMM launches while profiling: two uint64 per
// profile class (shader-clock ticks, 100 MHz ticks), one buffer per device,
// allocated when profiling is switched on.
std::map<int, unsigned long long*> g_prof_clk;

unsigned long long* prof_clk(int cls) {
  if (!g_prof.load(std::memory_order_relaxed)) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  auto it = g_prof_clk.find(dev);
  return it == g_prof_clk.end() ? nullptr : it->second + 2 * cls;
}

template <typename F>
hipError_t timed(int cls, hipStream_t s, F&& launch) {
  if (!g_prof.load(std::memory_order_relaxed)) return launch();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  g_prof_pending.push_back({cls, a, b});
  return hipSuccess;
}

// ---------------------------------------------------------------- counters
// Cumulative diagnostics (matopt_counters): plans built, device allocations
// and frees, bind launches.
enum { CNT_PLAN_BUILDS = 0, CNT_DEV_ALLOCS = 1, CNT_DEV_FREES = 2, CNT_BIND_LAUNCHES = 3 };
std::atomic<int64_t> g_counters[MATOPT_COUNTERS];

void bump(int k) { g_counters[k].fetch_add(1, std::memory_order_relaxed); }

// ---------------------------------------------------------------- plans
enum PlanKind {
  PK_NS = 2, PK_RMNP = 3, PK_COLCUT_PARTIAL = 4, PK_COLCUT_APPLY = 5, PK_ADAMW = 6
};

struct RmnpGroup {
  int wpr, nch, n;
  size_t off;  // byte offset of its task table in the plan buffer
};

// A GEMM stage's launch table and its length (the grid size of that stage:
// the three tables are packed separately and differ in length).
struct TileTable {
  size_t off = 0;   // byte offset in the plan buffer
  int n = 0;
  int uniform_k = 0;   // every tile has the same K extent (GemmParams::uniform_k)
};

// Everything a call's launches need that depends on the list of shapes only:
// descriptor templates (pointer fields empty, or byte offsets from the
// workspace / row-sum vector where BindMode says so) and the tile and task
// tables, in one device buffer, uploaded once.  No caller pointer is kept.
struct Plan {
  int device = -1;
  bool pooled = false;               // dbuf from the stream-ordered allocator
  void* dbuf = nullptr;
  std::vector<uint8_t> host;         // the uploaded bytes, kept until the plan is freed
  size_t o_tmpl = 0;                 // templates (MatDesc, or VecDesc for AdamW)
  size_t o_slot = 0;                 // descriptors of calls without a workspace
  size_t ws_desc = 0;                // Newton-Schulz plans: descriptor offset in the workspace
  size_t o_prep = 0;
  int n_prep = 0;     // prep tiles: prep_kernel's first, then prep_t_kernel's
  int n_prep_u = 0;   // prep_kernel's (all but transposed bf16 matrices)
  TileTable gram, poly, apply;
  int count = 0;
  std::vector<RmnpGroup> rmnp;
  // Calls that use this plan are enqueued one at a time and chained across
  // streams (a call on another stream than the previous one first waits, on
  // the device, for ev_last), so the descriptor slot is never rewritten under
  // a launch that still reads it and ev_last covers every use so far.
  std::mutex mu;
  hipEvent_t ev_last = nullptr;
  hipStream_t last_stream = nullptr;
  // Pointer values last written into the descriptor slot (kinds without a
  // workspace): a call with the same values finds them there already, in
  // stream order, and skips its bind launch.  Only compared, never used.
  std::vector<BindPtrs> slot_bound;

  template <class T>
  T* dev(size_t off) const { return (T*)((uint8_t*)dbuf + off); }
};

using PlanKey = std::vector<uint64_t>;
constexpr size_t kPlanCap = 64;
std::mutex g_plan_mu;
using PlanList = std::list<std::pair<PlanKey, std::shared_ptr<Plan>>>;
// Leaked singletons: no HIP call runs during static destruction.
PlanList& g_plans = *new PlanList();   // front = most recently used
std::vector<std::shared_ptr<Plan>>& g_retired = *new std::vector<std::shared_ptr<Plan>>();

// Frees evicted plans whose last use has completed on the device (polled,
// never waited for) and that no call still holds, stream-ordered on the
// caller's stream of the same device.
void sweep_retired(int dev, hipStream_t s) {
  for (size_t i = 0; i < g_retired.size();) {
    Plan& p = *g_retired[i];
    const bool idle = g_retired[i].use_count() == 1 &&
                      (!p.ev_last || hipEventQuery(p.ev_last) == hipSuccess);
    if (!idle || p.device != dev) {
      ++i;
      continue;
    }
    if (p.dbuf) {
      if (p.pooled) (void)hipFreeAsync(p.dbuf, s);
      else (void)hipFree(p.dbuf);
      bump(CNT_DEV_FREES);
    }
    if (p.ev_last) (void)hipEventDestroy(p.ev_last);
    g_retired.erase(g_retired.begin() + (long)i);
  }
}

struct HostBuf {
  std::vector<uint8_t> bytes;
  template <typename T>
  size_t put(const std::vector<T>& v) {
    size_t off = align256(bytes.size());
    bytes.resize(off + align256(v.size() * sizeof(T) + 1));
    if (!v.empty()) std::memcpy(bytes.data() + off, v.data(), v.size() * sizeof(T));
    return off;
  }
  size_t reserve(size_t n) {
    size_t off = align256(bytes.size());
    bytes.resize(off + align256(n + 1));
    return off;
  }
};

matopt_status hip_fail(const char* what, hipError_t e) {
  return fail(MATOPT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// One device buffer per plan from the stream-ordered allocator (the plain
// allocator if the device has no memory pools), filled from the plan's own
// host copy on `s`; ev_last marks the upload for calls on other streams.
matopt_status upload(Plan& p, hipStream_t s) {
  hipError_t e = hipEventCreateWithFlags(&p.ev_last, hipEventDisableTiming);
  if (e != hipSuccess) return hip_fail("plan event", e);
  e = hipMallocAsync(&p.dbuf, p.host.size(), s);
  p.pooled = e == hipSuccess;
  if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    e = hipMalloc(&p.dbuf, p.host.size());
  }
  if (e != hipSuccess) {
    p.dbuf = nullptr;
    return hip_fail("plan allocation", e);
  }
  bump(CNT_DEV_ALLOCS);
  e = hipMemcpyAsync(p.dbuf, p.host.data(), p.host.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(p.ev_last, s);
  if (e != hipSuccess) return hip_fail("plan upload", e);
  p.last_stream = s;
  return MATOPT_OK;
}

// The plan for `key`, built and uploaded on `s` if it is not cached.  Plans
// evicted beyond kPlanCap are retired and freed once idle (sweep_retired).
template <class Build>
matopt_status get_plan(const PlanKey& key, int dev, hipStream_t s, Build&& build,
                       std::shared_ptr<Plan>& out) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  sweep_retired(dev, s);
  for (auto it = g_plans.begin(); it != g_plans.end(); ++it)
    if (it->first == key) {
      g_plans.splice(g_plans.begin(), g_plans, it);
      out = g_plans.front().second;
      return MATOPT_OK;
    }
  auto p = std::make_shared<Plan>();
  p->device = dev;
  matopt_status st = build(*p);
  if (st != MATOPT_OK) return st;
  st = upload(*p, s);
  if (st != MATOPT_OK) {
    g_retired.push_back(p);   // whatever was allocated is freed once idle
    return st;
  }
  bump(CNT_PLAN_BUILDS);
  g_plans.emplace_front(key, p);
  while (g_plans.size() > kPlanCap) {
    g_retired.push_back(g_plans.back().second);
    g_plans.pop_back();
  }
  out = p;
  return MATOPT_OK;
}

// Holds a plan for one call's enqueue (see Plan::mu).
class PlanUse {
 public:
  PlanUse(Plan& p, hipStream_t s) : p_(p), s_(s) {
    p_.mu.lock();
    if (p_.last_stream != s_) err_ = hipStreamWaitEvent(s_, p_.ev_last, 0);
  }
  ~PlanUse() {
    (void)hipEventRecord(p_.ev_last, s_);
    p_.last_stream = s_;
    p_.mu.unlock();
  }
  hipError_t error() const { return err_; }

 private:
  Plan& p_;
  hipStream_t s_;
  hipError_t err_ = hipSuccess;
};

bool same_ptrs(const std::vector<BindPtrs>& a, const std::vector<BindPtrs>& b) {
  return a.size() == b.size() &&
         (a.empty() || std::memcmp(a.data(), b.data(), a.size() * sizeof(BindPtrs)) == 0);
}

// Writes descriptors [0, ptrs.size()) of `dst` from the templates and this
// call's pointers, kBindMax per launch.
matopt_status bind_descs(const void* tmpl, void* dst, const char* base, int mode,
                   const std::vector<BindPtrs>& ptrs, hipStream_t s) {
  BindArgs a;
  std::memset(&a, 0, sizeof(a));
  a.dst = dst;
  a.tmpl = tmpl;
  a.base = base;
  a.mode = mode;
  const int n = (int)ptrs.size();
  for (int first = 0; first < n; first += kBindMax) {
    a.first = first;
    a.n = std::min(kBindMax, n - first);
    for (int i = 0; i < a.n; ++i) a.ptr[i] = ptrs[first + i];
    hipError_t e = timed(10, s, [&] { return launch_bind(a, s); });
    if (e != hipSuccess) return hip_fail("bind launch", e);
    bump(CNT_BIND_LAUNCHES);
  }
  return MATOPT_OK;
}

template <class P>
P as_off(size_t off) {
  return (P)(uintptr_t)off;
}

// Templates and tile tables of a Newton-Schulz plan (muon step and NS only).
// The workspace-resident fields of the templates are byte offsets from the
// workspace (BIND_NS).
matopt_status build_ns_plan(Plan& P, int dt, const std::vector<Geo>& geo) {
  const int count = (int)geo.size();
  const Layout L = layout(geo, dt);
  // GEMM output tile: the padding granule for bf16, a divisor of it for float32
  const int tile = sdt(dt) == DT_BF16 ? kTileBf16 : kGridF32;
  std::vector<MatDesc> mats(count);
  std::vector<PrepTile> prep;
  std::vector<TileUnit> u3, u4, u5;
  prep.reserve(L.n_prep);
  for (int i = 0; i < count; ++i) {
    const Geo& g = geo[i];
    MatDesc& d = mats[i];
    std::memset(&d, 0, sizeof(d));
    d.rows = g.rows;
    d.cols = g.cols;
    d.m = g.m;
    d.n = g.n;
    d.mp = g.mp;
    d.np = g.np;
    d.transposed = g.transposed ? 1 : 0;
    d.vec_ok = (g.cols % (16 / esize(dt))) == 0 ? 1 : 0;
    d.upd_scale = (float)std::sqrt(std::max(1.0, (double)g.rows / (double)g.cols));
    d.prep_tiles_c = g.prep_tc;
    d.x[0] = as_off<void*>(L.x0[i]);
    d.x[1] = as_off<void*>(L.x1[i]);
    // X0 is the stored V; when V has X0's layout the first iteration reads it
    // in place and the prep kernel skips the copy (bind sets x0in)
    d.x0_is_v = (sdt(dt) == DT_BF16 && !g.transposed && g.rows == g.mp && g.cols == g.np) ? 1 : 0;
    d.a = as_off<void*>(L.a[i]);
    d.b = as_off<void*>(L.b[i]);
    d.xs = as_off<float*>(L.xs + 4 * (size_t)i);
    d.partials = as_off<float*>(L.partials + 4 * (size_t)L.prep_off[i]);
    d.n_prep = g.prep_tr * g.prep_tc;
    if (!(g.transposed && sdt(dt) == DT_BF16)) {
      int idx = 0;
      for (int tr = 0; tr < g.prep_tr; ++tr)
        for (int tc = 0; tc < g.prep_tc; ++tc) prep.push_back({i, tr, tc, idx++});
    }
    const int tm = g.mp / tile, tn = g.np / tile;
    // diagonal tiles as the GEMM build treats them (bf16: 36 of their 64
    // blocks; the Gram's two per workgroup, in step with the matrix's other
    // tiles, which share their operand panels through L2)
    const int dm3 = sdt(dt) == DT_BF16 ? gemm_bf16_diag_mode(0) : 0;
    const int dm4 = sdt(dt) == DT_BF16 ? gemm_bf16_diag_mode(1) : 0;
    units_triangle(i, tm, g.np, u3, dm3 ? 9 : 16, dm3 == 2);
    units_triangle(i, tm, g.mp, u4, dm4 ? 9 : 16, dm4 == 2);
    units_full(i, tm, tn, g.mp, u5);
  }
  // the transposed bf16 matrices' tiles, for their own launch
  P.n_prep_u = (int)prep.size();
  for (int i = 0; i < count; ++i) {
    const Geo& g = geo[i];
    if (!(g.transposed && sdt(dt) == DT_BF16)) continue;
    int idx = 0;
    for (int tr = 0; tr < g.prep_tr; ++tr)
      for (int tc = 0; tc < g.prep_tc; ++tc) prep.push_back({i, tr, tc, idx++});
  }
  static_assert(sizeof(TileRef) == sizeof(GemmTile), "tile record layout");
  const std::vector<TileRef> k3 = xcd_schedule(u3), k4 = xcd_schedule(u4), k5 = xcd_schedule(u5);

  HostBuf hb;
  P.o_tmpl = hb.put(mats);
  const size_t o_prep = hb.put(prep);
  const size_t o_k3 = hb.put(k3);
  const size_t o_k4 = hb.put(k4);
  const size_t o_k5 = hb.put(k5);
  P.host = std::move(hb.bytes);
  P.count = count;
  P.n_prep = (int)prep.size();
  P.ws_desc = L.desc;
  P.o_prep = o_prep;
  P.gram = TileTable{o_k3, (int)k3.size()};
  P.poly = TileTable{o_k4, (int)k4.size()};
  bool same_k = true;
  for (const Geo& g : geo) same_k = same_k && g.mp == geo[0].mp;
  P.apply = TileTable{o_k5, (int)k5.size(), same_k ? 1 : 0};
  return MATOPT_OK;
}

matopt_status build_rmnp_plan(Plan& P, int dt, const std::vector<std::pair<int64_t, int64_t>>& shp) {
  const int count = (int)shp.size();
  const int E = 16 / esize(dt);
  std::vector<MatDesc> descs(count);
  std::map<std::pair<int, int>, std::vector<RmnpTask>> groups;
  for (int i = 0; i < count; ++i) {
    MatDesc& d = descs[i];
    std::memset(&d, 0, sizeof(d));
    d.rows = shp[i].first;
    d.cols = shp[i].second;
    d.upd_scale = (float)std::sqrt(std::max(1.0, (double)d.rows / (double)d.cols));
    const bool vec = d.cols % E == 0;
    const int64_t nchunks = d.cols / E;
    int wpr = 4, nch = 0;
    // one wave per row up to 512 chunks; wider rows take a whole workgroup
    // (fewer registers per lane, more waves in flight: measured ~1% faster)
    if (vec && nchunks <= 64 * 8) {
      wpr = 1;
      for (int c : {1, 2, 4, 8, 16})
        if (64 * c >= nchunks) { nch = c; break; }
    } else if (vec && nchunks <= 256 * 16) {
      wpr = 4;
      for (int c : {4, 8, 16})
        if (256 * c >= nchunks) { nch = c; break; }
    }
    auto& tasks = groups[{wpr, nch}];
    const int step = (wpr == 1 && nch > 0) ? 4 : 1;
    for (int64_t r = 0; r < d.rows; r += step) tasks.push_back({i, (int32_t)r});
  }
  HostBuf hb;
  P.o_tmpl = hb.put(descs);
  P.o_slot = hb.reserve(descs.size() * sizeof(MatDesc));
  for (auto& kv : groups) {
    RmnpGroup g;
    g.wpr = kv.first.first;
    g.nch = kv.first.second;
    g.n = (int)kv.second.size();
    g.off = hb.put(kv.second);
    P.rmnp.push_back(g);
  }
  P.host = std::move(hb.bytes);
  P.count = count;
  return MATOPT_OK;
}

// Where the tables of a Newton-Schulz plan are on the device: the plan's own
// buffer, or the allocation-free entry point's scratch copy of it.
struct NsTables {
  const uint8_t* base;
  size_t o_prep;
  int n_prep, n_prep_u, count;
  TileTable gram, poly, apply;
  NsTables(const Plan& p, const void* dev_base)
      : base((const uint8_t*)dev_base), o_prep(p.o_prep), n_prep(p.n_prep),
        n_prep_u(p.n_prep_u), count(p.count),
        gram(p.gram), poly(p.poly), apply(p.apply) {}
  template <class T>
  const T* dev(size_t off) const { return (const T*)(base + off); }
};

// Enqueue the Newton-Schulz pipeline on descriptors `mats` (this call's,
// already bound) with the tables of P.
matopt_status run_ns(const NsTables& P, const MatDesc* mats, int dt, bool momentum, float mu,
                     float lr, double wdl, int ns_steps, float a, float b, float c, float eps,
                     int out_kind, int out_dt, hipStream_t s) {
  hipError_t e;
  const bool split = dt == DT_BF16_SPLIT;
  dt = sdt(dt);
  const PrepTile* prep = P.dev<const PrepTile>(P.o_prep);
  PrepParams pp{mats, prep, mu, momentum ? 1 : 0};
  e = timed(0, s, [&] { return launch_prep(dt, pp, P.n_prep_u, s); });
  if (e != hipSuccess) return hip_fail("prep launch", e);
  if (P.n_prep > P.n_prep_u) {
    const PrepParams pt{mats, prep + P.n_prep_u, mu, momentum ? 1 : 0};
    e = timed(0, s, [&] { return launch_prep_t(pt, P.n_prep - P.n_prep_u, s); });
    if (e != hipSuccess) return hip_fail("prep launch", e);
  }
  FinalizeParams fp{mats, eps};
  e = timed(1, s, [&] { return launch_finalize(fp, P.count, s); });
  if (e != hipSuccess) return hip_fail("finalize launch", e);
  // every stage launches exactly its own table
  auto gemm = [&](GemmParams g, const TileTable& t) {
    g.tiles = P.dev<const GemmTile>(t.off);
    g.uniform_k = t.uniform_k;
    return dt == DT_BF16 ? launch_gemm_bf16(g, t.n, s) : launch_gemm_f32(g, t.n, s);
  };
  for (int it = 0; it < ns_steps; ++it) {
    GemmParams g;
    std::memset(&g, 0, sizeof(g));
    g.mats = mats;
    g.cur = it & 1;
    g.first = it == 0 ? 1 : 0;
    g.out_dt = out_dt;
    g.a = a;
    g.b = b;
    g.c = c;
    g.lr = lr;
    g.wdl = wdl;
    g.split = split ? 1 : 0;
    g.stage = 0;
    g.out_kind = OUT_NEXT_X;
    g.clk = dt == DT_BF16 ? prof_clk(2) : nullptr;
    e = timed(2, s, [&] { return gemm(g, P.gram); });
    if (e != hipSuccess) return hip_fail("gram launch", e);
    g.stage = 1;
    g.clk = dt == DT_BF16 ? prof_clk(3) : nullptr;
    e = timed(3, s, [&] { return gemm(g, P.poly); });
    if (e != hipSuccess) return hip_fail("poly launch", e);
    g.stage = 2;
    g.out_kind = it == ns_steps - 1 ? out_kind : OUT_NEXT_X;
    g.clk = dt == DT_BF16 ? prof_clk(4) : nullptr;
    e = timed(4, s, [&] { return gemm(g, P.apply); });
    if (e != hipSuccess) return hip_fail("apply launch", e);
  }
  if (ns_steps == 0) {
    ScaleOutParams sp{mats, prep, out_kind, out_dt, lr, wdl};
    e = timed(5, s, [&] { return launch_scale_out(dt, sp, P.n_prep, s); });
    if (e != hipSuccess) return hip_fail("scale_out launch", e);
  }
  return MATOPT_OK;
}

// Plan lookup, binding and the Newton-Schulz pipeline of one muon / NS call
// (arguments already validated).
matopt_status ns_call(int dt, const std::vector<Geo>& geo, const std::vector<BindPtrs>& ptrs,
                      void* workspace, int dev, hipStream_t s, bool momentum, float mu, float lr,
                      double wdl, int ns_steps, float a, float b, float c, float eps,
                      int out_kind, int out_dt) {
  PlanKey key{PK_NS, (uint64_t)dt, (uint64_t)dev, (uint64_t)geo.size()};
  for (const Geo& g : geo) {
    key.push_back((uint64_t)g.rows);
    key.push_back((uint64_t)g.cols);
  }
  std::shared_ptr<Plan> plan;
  matopt_status st =
      get_plan(key, dev, s, [&](Plan& p) { return build_ns_plan(p, dt, geo); }, plan);
  if (st != MATOPT_OK) return st;
  PlanUse use(*plan, s);
  if (use.error() != hipSuccess) return hip_fail("plan stream wait", use.error());
  MatDesc* mats = (MatDesc*)((uint8_t*)workspace + plan->ws_desc);
  if ((st = bind_descs(plan->dev<MatDesc>(plan->o_tmpl), mats, (const char*)workspace, BIND_NS, ptrs,
                 s)) != MATOPT_OK)
    return st;
  return run_ns(NsTables(*plan, plan->dbuf), mats, dt, momentum, mu, lr, wdl, ns_steps, a, b, c,
                eps, out_kind, out_dt, s);
}

matopt_status check_common(int32_t count, int dt, bool ns_entry = false) {
  if (count < 0) return fail(MATOPT_ERR_PARAM, "count < 0");
  if (ns_entry && dt == DT_BF16_SPLIT) return MATOPT_OK;
  if (dt != DT_F32 && dt != DT_BF16)
    return fail(MATOPT_ERR_DTYPE, ns_entry ? "dtype must be MATOPT_F32, MATOPT_BF16 or MATOPT_BF16_SPLIT"
                                           : "dtype must be MATOPT_F32 or MATOPT_BF16");
  return MATOPT_OK;
}

matopt_status check_ns_params(int32_t ns_steps, float a, float b, float c, float eps) {
  if (ns_steps < 0 || ns_steps > 64) return fail(MATOPT_ERR_PARAM, "ns_steps outside [0, 64]");
  if (!finite(a) || !finite(b) || !finite(c)) return fail(MATOPT_ERR_PARAM, "non-finite Newton-Schulz coefficient");
  if (!finite(eps) || eps < 0.f) return fail(MATOPT_ERR_PARAM, "eps must be finite and >= 0");
  return MATOPT_OK;
}

// Column-cut RMNP plan: templates whose `partials` are byte offsets into the
// caller's row-sum vector (matrix i starts after the rows before it) and one
// task per 4 rows.  full_cols (NULL: the slice's own width) sets the update
// scale from the whole matrix's shape.
matopt_status build_colcut_plan(Plan& P, int dt, const matopt_mat* mats, int count,
                                const int64_t* full_cols) {
  const int E = 16 / esize(dt);
  std::vector<MatDesc> descs(count);
  std::vector<RmnpTask> tasks;
  int64_t off = 0;
  for (int i = 0; i < count; ++i) {
    MatDesc& d = descs[i];
    std::memset(&d, 0, sizeof(d));
    d.rows = mats[i].rows;
    d.cols = mats[i].cols;
    const int64_t fc = full_cols ? full_cols[i] : d.cols;
    d.upd_scale = (float)std::sqrt(std::max(1.0, (double)d.rows / (double)fc));
    d.vec_ok = d.cols % E == 0 ? 1 : 0;
    d.partials = as_off<float*>((size_t)off * 4);
    off += d.rows;
    for (int64_t r = 0; r < d.rows; r += 4) tasks.push_back({i, (int32_t)r});
  }
  HostBuf hb;
  P.o_tmpl = hb.put(descs);
  P.o_slot = hb.reserve(descs.size() * sizeof(MatDesc));
  RmnpGroup g;
  g.wpr = 1;
  g.nch = 0;
  g.n = (int)tasks.size();
  g.off = hb.put(tasks);
  P.rmnp.push_back(g);
  P.host = std::move(hb.bytes);
  P.count = count;
  return MATOPT_OK;
}

// Shared by both column-cut halves: validation, plan lookup, bind, one launch.
matopt_status colcut_run(bool apply, const matopt_mat* mats, int32_t count, matopt_dtype dt,
                         float mu, float lr, float eps, const float* rowsq,
                         const int64_t* full_cols, void* stream) {
  matopt_status st = check_common(count, dt);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!mats) return fail(MATOPT_ERR_NULL, "mats is NULL");
  if (!rowsq) return fail(MATOPT_ERR_NULL, "rowsq is NULL");
  if (((uintptr_t)rowsq & 3) != 0) return fail(MATOPT_ERR_ALIGN, "rowsq not 4-byte aligned");
  if (!finite(mu) || !finite(lr) || !finite(eps) || eps < 0.f)
    return fail(MATOPT_ERR_PARAM, "non-finite mu/lr/eps or eps < 0");
  std::vector<Span> spans;
  const size_t es = esize(dt);
  int64_t total_rows = 0;
  std::vector<BindPtrs> ptrs(count);
  for (int i = 0; i < count; ++i) {
    const matopt_mat& m = mats[i];
    const std::string tag = "matrix " + std::to_string(i);
    void* a = apply ? m.w : const_cast<void*>(m.g);   // the other operand of this half
    if (!a || !m.v) return fail(MATOPT_ERR_NULL, tag + ": NULL pointer");
    if ((st = check_shape(m.rows, m.cols, i)) != MATOPT_OK) return st;
    if (apply && full_cols && (full_cols[i] < m.cols || full_cols[i] > kMaxSide))
      return fail(MATOPT_ERR_SHAPE, tag + ": full_cols smaller than the slice or too large");
    if (!aligned16(a) || !aligned16(m.v)) return fail(MATOPT_ERR_ALIGN, tag + ": pointer not 16-byte aligned");
    const size_t bytes = (size_t)m.rows * m.cols * es;
    spans.push_back({(uintptr_t)a, (uintptr_t)a + bytes, tag + (apply ? " W" : " G")});
    spans.push_back({(uintptr_t)m.v, (uintptr_t)m.v + bytes, tag + " V"});
    total_rows += m.rows;
    ptrs[i] = BindPtrs{{apply ? m.w : nullptr, apply ? nullptr : m.g, m.v, nullptr}};
  }
  spans.push_back({(uintptr_t)rowsq, (uintptr_t)rowsq + (size_t)total_rows * 4, "rowsq"});
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{(uint64_t)(apply ? PK_COLCUT_APPLY : PK_COLCUT_PARTIAL), (uint64_t)dt, (uint64_t)dev,
              (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)mats[i].rows);
    key.push_back((uint64_t)mats[i].cols);
    key.push_back((uint64_t)(apply && full_cols ? full_cols[i] : mats[i].cols));
  }
  std::shared_ptr<Plan> plan;
  st = get_plan(key, dev, s, [&](Plan& p) {
    return build_colcut_plan(p, dt, mats, count, apply ? full_cols : nullptr);
  }, plan);
  if (st != MATOPT_OK) return st;
  PlanUse use(*plan, s);
  if (use.error() != hipSuccess) return hip_fail("plan stream wait", use.error());
  MatDesc* slot = plan->dev<MatDesc>(plan->o_slot);
  // the row-sum vector is part of what the descriptors hold
  ptrs.push_back(BindPtrs{{rowsq, nullptr, nullptr, nullptr}});
  if (!same_ptrs(ptrs, plan->slot_bound)) {
    plan->slot_bound.clear();
    const std::vector<BindPtrs> mats_only(ptrs.begin(), ptrs.end() - 1);
    if ((st = bind_descs(plan->dev<MatDesc>(plan->o_tmpl), slot, (const char*)rowsq, BIND_COLCUT,
                         mats_only, s)) != MATOPT_OK)
      return st;
    plan->slot_bound = ptrs;
  }
  const RmnpGroup& g = plan->rmnp[0];
  ColcutParams cp{slot, plan->dev<RmnpTask>(g.off), mu, lr, eps};
  hipError_t e = timed(apply ? 8 : 7, s, [&] { return launch_colcut(dt, apply, cp, g.n, s); });
  if (e != hipSuccess) return hip_fail(apply ? "colcut apply launch" : "colcut partial launch", e);
  return MATOPT_OK;
}

// AdamW plan: one template per tensor and one task per kAdamwTask elements.
matopt_status build_adamw_plan(Plan& P, const matopt_vec* vecs, int count) {
  std::vector<VecDesc> descs(count);
  std::vector<VecTask> tasks;
  for (int i = 0; i < count; ++i) {
    descs[i] = VecDesc{nullptr, nullptr, nullptr, nullptr, vecs[i].n};
    for (int64_t e = 0; e < vecs[i].n; e += kAdamwTask) tasks.push_back({i, 0, e});
  }
  HostBuf hb;
  P.o_tmpl = hb.put(descs);
  P.o_slot = hb.reserve(descs.size() * sizeof(VecDesc));
  RmnpGroup g;
  g.wpr = 0;
  g.nch = 0;
  g.n = (int)tasks.size();
  g.off = hb.put(tasks);
  P.rmnp.push_back(g);
  P.host = std::move(hb.bytes);
  P.count = count;
  return MATOPT_OK;
}

// Validation of a muon / NS workspace against the layout of `geo`.
matopt_status check_workspace(const std::vector<Geo>& geo, int dt, void* workspace,
                              size_t workspace_bytes, std::vector<Span>& spans) {
  const size_t need = layout(geo, dt).total;
  if (!workspace || workspace_bytes < need)
    return fail(MATOPT_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                          std::to_string(workspace ? workspace_bytes : 0));
  if (((uintptr_t)workspace & 255) != 0) return fail(MATOPT_ERR_ALIGN, "workspace not 256-byte aligned");
  spans.push_back({(uintptr_t)workspace, (uintptr_t)workspace + need, "workspace"});
  return check_overlap(spans);
}

}  // namespace

// ==================================================================== C ABI
extern "C" {

int32_t matopt_version(void) { return 10100; }

const char* matopt_status_string(matopt_status s) {
  switch (s) {
    case MATOPT_OK: return "MATOPT_OK";
    case MATOPT_ERR_NULL: return "MATOPT_ERR_NULL";
    case MATOPT_ERR_SHAPE: return "MATOPT_ERR_SHAPE";
    case MATOPT_ERR_DTYPE: return "MATOPT_ERR_DTYPE";
    case MATOPT_ERR_PARAM: return "MATOPT_ERR_PARAM";
    case MATOPT_ERR_WORKSPACE: return "MATOPT_ERR_WORKSPACE";
    case MATOPT_ERR_ALIAS: return "MATOPT_ERR_ALIAS";
    case MATOPT_ERR_ALIGN: return "MATOPT_ERR_ALIGN";
    case MATOPT_ERR_DEVICE: return "MATOPT_ERR_DEVICE";
    case MATOPT_ERR_HIP: return "MATOPT_ERR_HIP";
    case MATOPT_ERR_INTERNAL: return "MATOPT_ERR_INTERNAL";
  }
  return "MATOPT_ERR_UNKNOWN";
}

const char* matopt_last_error_detail(void) { return g_detail.c_str(); }

size_t matopt_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t count,
                              matopt_dtype dt) {
  if (count < 0 || (count > 0 && (!rows || !cols))) return 0;
  if (dt != MATOPT_F32 && dt != MATOPT_BF16 && dt != DT_BF16_SPLIT) return 0;
  std::vector<Geo> geo;
  for (int i = 0; i < count; ++i) {
    if (check_shape(rows[i], cols[i], i) != MATOPT_OK) return 0;
    geo.push_back(geometry(rows[i], cols[i], dt));
  }
  return layout(geo, dt).total;
}

}  // extern "C"

// The Muon step with decoupled weight decay wd (0: the plain step).
static matopt_status muon_impl(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                               float mu, float lr, float wd, int32_t ns_steps, float a,
                               float b, float c, float eps, void* workspace,
                               size_t workspace_bytes, void* stream) {
  matopt_status st = check_common(count, dt, true);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!mats) return fail(MATOPT_ERR_NULL, "mats is NULL");
  if (!finite(mu) || !finite(lr)) return fail(MATOPT_ERR_PARAM, "non-finite mu or lr");
  if (!finite(wd)) return fail(MATOPT_ERR_PARAM, "non-finite weight decay");
  if ((st = check_ns_params(ns_steps, a, b, c, eps)) != MATOPT_OK) return st;
  std::vector<Geo> geo;
  std::vector<Span> spans;
  std::vector<BindPtrs> ptrs(count);
  const size_t es = esize(dt);
  for (int i = 0; i < count; ++i) {
    const matopt_mat& m = mats[i];
    if (!m.w || !m.g || !m.v) return fail(MATOPT_ERR_NULL, "matrix " + std::to_string(i) + ": NULL pointer");
    if ((st = check_shape(m.rows, m.cols, i)) != MATOPT_OK) return st;
    if (!aligned16(m.w) || !aligned16(m.g) || !aligned16(m.v))
      return fail(MATOPT_ERR_ALIGN, "matrix " + std::to_string(i) + ": pointer not 16-byte aligned");
    const size_t bytes = (size_t)m.rows * m.cols * es;
    const std::string tag = "matrix " + std::to_string(i);
    spans.push_back({(uintptr_t)m.w, (uintptr_t)m.w + bytes, tag + " W"});
    spans.push_back({(uintptr_t)m.g, (uintptr_t)m.g + bytes, tag + " G"});
    spans.push_back({(uintptr_t)m.v, (uintptr_t)m.v + bytes, tag + " V"});
    geo.push_back(geometry(m.rows, m.cols, dt));
    ptrs[i] = BindPtrs{{m.w, m.g, m.v, nullptr}};
  }
  if ((st = check_workspace(geo, dt, workspace, workspace_bytes, spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  const double wdl = (double)lr * (double)wd;   // exact: a product of two floats
  return ns_call(dt, geo, ptrs, workspace, dev, (hipStream_t)stream, true, mu, lr, wdl, ns_steps,
                 a, b, c, eps, OUT_W_UPDATE, sdt(dt));
}

// ------------------------------------------------------ allocation-free step
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation):
// muon_step_batched_noalloc keeps its workspace and its plan tables in this
// file-scope array instead -- one copy per GPU the library runs on, held
// until the process ends.  In host code `scratch` only names the array; the
// device address of a GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and is what every launch receives.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;   // held for the whole enqueue of one call
std::map<int, uint8_t*>& g_scratch_ptr = *new std::map<int, uint8_t*>();
// host-side tables of the allocation-free entry point (host memory only)
PlanList& g_na_plans = *new PlanList();
constexpr size_t kNaPlanCap = 16;

// Device address of the current device's copy of `scratch` (g_scratch_mu held).
matopt_status scratch_address(int dev, uint8_t** out) {
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail("scratch symbol address", e);
    it = g_scratch_ptr.emplace(dev, (uint8_t*)p).first;
  }
  *out = it->second;
  return MATOPT_OK;
}

// Copies `bytes` to dst on s through kernel arguments, kUploadBytes per launch.
matopt_status upload_args(uint8_t* dst, const std::vector<uint8_t>& bytes, hipStream_t s) {
  UploadArgs a;
  std::memset(&a, 0, sizeof(a));
  for (size_t off = 0; off < bytes.size(); off += kUploadBytes) {
    const size_t n = std::min(bytes.size() - off, (size_t)kUploadBytes);
    a.dst = dst + off;
    a.n = (uint32_t)n;
    std::memcpy(a.data, bytes.data() + off, n);
    hipError_t e = launch_upload(a, s);
    if (e != hipSuccess) return hip_fail("table upload launch", e);
  }
  return MATOPT_OK;
}

// Host tables for `key` (built once; g_scratch_mu held).
const Plan& na_plan(const PlanKey& key, int dt, const std::vector<Geo>& geo) {
  for (auto it = g_na_plans.begin(); it != g_na_plans.end(); ++it)
    if (it->first == key) {
      g_na_plans.splice(g_na_plans.begin(), g_na_plans, it);
      return *g_na_plans.front().second;
    }
  auto p = std::make_shared<Plan>();
  (void)build_ns_plan(*p, dt, geo);
  g_na_plans.emplace_front(key, p);
  while (g_na_plans.size() > kNaPlanCap) g_na_plans.pop_back();
  return *p;
}

}  // namespace

extern "C" {

matopt_status muon_step_batched_noalloc(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                        float mu, float lr, int32_t ns_steps, float a, float b,
                                        float c, float eps, void* stream) {
  matopt_status st = check_common(count, dt, true);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!mats) return fail(MATOPT_ERR_NULL, "mats is NULL");
  if (!finite(mu) || !finite(lr)) return fail(MATOPT_ERR_PARAM, "non-finite mu or lr");
  if ((st = check_ns_params(ns_steps, a, b, c, eps)) != MATOPT_OK) return st;
  std::vector<Geo> geo;
  std::vector<Span> spans;
  std::vector<BindPtrs> ptrs(count);
  const size_t es = esize(dt);
  PlanKey key{PK_NS, (uint64_t)dt, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    const matopt_mat& m = mats[i];
    if (!m.w || !m.g || !m.v) return fail(MATOPT_ERR_NULL, "matrix " + std::to_string(i) + ": NULL pointer");
    if ((st = check_shape(m.rows, m.cols, i)) != MATOPT_OK) return st;
    if (!aligned16(m.w) || !aligned16(m.g) || !aligned16(m.v))
      return fail(MATOPT_ERR_ALIGN, "matrix " + std::to_string(i) + ": pointer not 16-byte aligned");
    const size_t bytes = (size_t)m.rows * m.cols * es;
    const std::string tag = "matrix " + std::to_string(i);
    spans.push_back({(uintptr_t)m.w, (uintptr_t)m.w + bytes, tag + " W"});
    spans.push_back({(uintptr_t)m.g, (uintptr_t)m.g + bytes, tag + " G"});
    spans.push_back({(uintptr_t)m.v, (uintptr_t)m.v + bytes, tag + " V"});
    geo.push_back(geometry(m.rows, m.cols, dt));
    ptrs[i] = BindPtrs{{m.w, m.g, m.v, nullptr}};
    key.push_back((uint64_t)m.rows);
    key.push_back((uint64_t)m.cols);
  }
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  const size_t ws_bytes = layout(geo, dt).total;   // a multiple of 256
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  const Plan& plan = na_plan(key, dt, geo);
  const size_t need = ws_bytes + plan.host.size();
  if (need > kScratchBytes)
    return fail(MATOPT_ERR_WORKSPACE, "this list of shapes needs " + std::to_string(need) +
                                          " bytes of device scratch; the allocation-free step has " +
                                          std::to_string(kScratchBytes));
  uint8_t* base = nullptr;
  if ((st = scratch_address(dev, &base)) != MATOPT_OK) return st;
  uint8_t* tables = base + ws_bytes;
  if ((st = upload_args(tables, plan.host, s)) != MATOPT_OK) return st;
  MatDesc* descs = (MatDesc*)(base + plan.ws_desc);
  if ((st = bind_descs(tables + plan.o_tmpl, descs, (const char*)base, BIND_NS, ptrs, s)) !=
      MATOPT_OK)
    return st;
  return run_ns(NsTables(plan, tables), descs, dt, true, mu, lr, 0.0, ns_steps, a, b, c, eps,
                OUT_W_UPDATE, sdt(dt), s);
}

}  // extern "C"

extern "C" {

matopt_status muon_step_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                float mu, float lr, int32_t ns_steps, float a, float b,
                                float c, float eps, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return muon_impl(mats, count, dt, mu, lr, 0.f, ns_steps, a, b, c, eps, workspace,
                   workspace_bytes, stream);
}

matopt_status muon_step_batched_wd(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                   float mu, float lr, float wd, int32_t ns_steps, float a,
                                   float b, float c, float eps, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return muon_impl(mats, count, dt, mu, lr, wd, ns_steps, a, b, c, eps, workspace,
                   workspace_bytes, stream);
}

matopt_status ns_orthogonalize_batched(const void* const* x, void* const* o, const int64_t* rows,
                                       const int64_t* cols, int32_t count, matopt_dtype in_dt,
                                       matopt_dtype out_dt, int32_t ns_steps, float a, float b,
                                       float c, float eps, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  matopt_status st = check_common(count, in_dt, true);
  if (st != MATOPT_OK) return st;
  if (out_dt != MATOPT_F32 && out_dt != MATOPT_BF16) return fail(MATOPT_ERR_DTYPE, "invalid out_dt");
  if (count == 0) return MATOPT_OK;
  if (!x || !o || !rows || !cols) return fail(MATOPT_ERR_NULL, "NULL argument array");
  if ((st = check_ns_params(ns_steps, a, b, c, eps)) != MATOPT_OK) return st;
  std::vector<Geo> geo;
  std::vector<Span> spans;
  std::vector<BindPtrs> ptrs(count);
  const size_t es_in = esize(in_dt), es_out = esize(out_dt);
  for (int i = 0; i < count; ++i) {
    if (!x[i] || !o[i]) return fail(MATOPT_ERR_NULL, "matrix " + std::to_string(i) + ": NULL pointer");
    if ((st = check_shape(rows[i], cols[i], i)) != MATOPT_OK) return st;
    if (!aligned16(x[i]) || !aligned16(o[i]))
      return fail(MATOPT_ERR_ALIGN, "matrix " + std::to_string(i) + ": pointer not 16-byte aligned");
    const size_t n = (size_t)rows[i] * cols[i];
    const std::string tag = "matrix " + std::to_string(i);
    spans.push_back({(uintptr_t)x[i], (uintptr_t)x[i] + n * es_in, tag + " x"});
    spans.push_back({(uintptr_t)o[i], (uintptr_t)o[i] + n * es_out, tag + " o"});
    geo.push_back(geometry(rows[i], cols[i], in_dt));
    ptrs[i] = BindPtrs{{nullptr, nullptr, x[i], o[i]}};
  }
  if ((st = check_workspace(geo, in_dt, workspace, workspace_bytes, spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  return ns_call(in_dt, geo, ptrs, workspace, dev, (hipStream_t)stream, false, 0.f, 0.f, 0.0,
                 ns_steps, a, b, c, eps, OUT_O, out_dt);
}

matopt_status rmnp_step_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt, float mu,
                                float lr, float eps, void* stream) {
  matopt_status st = check_common(count, dt);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!mats) return fail(MATOPT_ERR_NULL, "mats is NULL");
  if (!finite(mu) || !finite(lr) || !finite(eps) || eps < 0.f)
    return fail(MATOPT_ERR_PARAM, "non-finite mu/lr/eps or eps < 0");
  std::vector<Span> spans;
  std::vector<BindPtrs> ptrs(count);
  std::vector<std::pair<int64_t, int64_t>> shp(count);
  const size_t es = esize(dt);
  for (int i = 0; i < count; ++i) {
    const matopt_mat& m = mats[i];
    if (!m.w || !m.g || !m.v) return fail(MATOPT_ERR_NULL, "matrix " + std::to_string(i) + ": NULL pointer");
    if ((st = check_shape(m.rows, m.cols, i)) != MATOPT_OK) return st;
    if (!aligned16(m.w) || !aligned16(m.g) || !aligned16(m.v))
      return fail(MATOPT_ERR_ALIGN, "matrix " + std::to_string(i) + ": pointer not 16-byte aligned");
    const size_t bytes = (size_t)m.rows * m.cols * es;
    const std::string tag = "matrix " + std::to_string(i);
    spans.push_back({(uintptr_t)m.w, (uintptr_t)m.w + bytes, tag + " W"});
    spans.push_back({(uintptr_t)m.g, (uintptr_t)m.g + bytes, tag + " G"});
    spans.push_back({(uintptr_t)m.v, (uintptr_t)m.v + bytes, tag + " V"});
    ptrs[i] = BindPtrs{{m.w, m.g, m.v, nullptr}};
    shp[i] = {m.rows, m.cols};
  }
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{PK_RMNP, (uint64_t)dt, (uint64_t)dev, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)mats[i].rows);
    key.push_back((uint64_t)mats[i].cols);
  }
  std::shared_ptr<Plan> plan;
  st = get_plan(key, dev, s, [&](Plan& p) { return build_rmnp_plan(p, dt, shp); }, plan);
  if (st != MATOPT_OK) return st;
  PlanUse use(*plan, s);
  if (use.error() != hipSuccess) return hip_fail("plan stream wait", use.error());
  MatDesc* slot = plan->dev<MatDesc>(plan->o_slot);
  if (!same_ptrs(ptrs, plan->slot_bound)) {
    plan->slot_bound.clear();
    if ((st = bind_descs(plan->dev<MatDesc>(plan->o_tmpl), slot, nullptr, BIND_ROWS, ptrs, s)) !=
        MATOPT_OK)
      return st;
    plan->slot_bound = ptrs;
  }
  RmnpParams rp{slot, nullptr, mu, lr, eps};
  for (const RmnpGroup& g : plan->rmnp) {
    rp.tasks = plan->dev<RmnpTask>(g.off);
    hipError_t e = timed(6, s, [&] { return launch_rmnp(dt, g.wpr, g.nch, rp, g.n, s); });
    if (e != hipSuccess) return hip_fail("rmnp launch", e);
  }
  return MATOPT_OK;
}

matopt_status rmnp_colcut_partial_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                          float mu, float* rowsq, void* stream) {
  return colcut_run(false, mats, count, dt, mu, 0.f, 0.f, rowsq, nullptr, stream);
}

matopt_status rmnp_colcut_apply_batched(const matopt_mat* mats, int32_t count, matopt_dtype dt,
                                        float lr, float eps, const float* rowsq,
                                        const int64_t* full_cols, void* stream) {
  return colcut_run(true, mats, count, dt, 0.f, lr, eps, rowsq, full_cols, stream);
}

matopt_status adamw_step_batched(const matopt_vec* vecs, int32_t count, matopt_dtype dt, float lr,
                                 float beta1, float beta2, float eps, float wd, int32_t step,
                                 void* stream) {
  matopt_status st = check_common(count, dt);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!vecs) return fail(MATOPT_ERR_NULL, "vecs is NULL");
  if (!finite(lr) || !finite(wd) || !finite(eps) || eps < 0.f)
    return fail(MATOPT_ERR_PARAM, "non-finite lr/wd/eps or eps < 0");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
    return fail(MATOPT_ERR_PARAM, "betas must lie in [0, 1)");
  if (step < 1) return fail(MATOPT_ERR_PARAM, "step must be >= 1");
  std::vector<Span> spans;
  std::vector<BindPtrs> ptrs(count);
  const size_t es = esize(dt);
  for (int i = 0; i < count; ++i) {
    const matopt_vec& t = vecs[i];
    const std::string tag = "tensor " + std::to_string(i);
    if (!t.p || !t.g || !t.m || !t.v) return fail(MATOPT_ERR_NULL, tag + ": NULL pointer");
    if (t.n < 1 || t.n > kMaxElems) return fail(MATOPT_ERR_SHAPE, tag + ": invalid length");
    if (!aligned16(t.p) || !aligned16(t.g) || !aligned16(t.m) || !aligned16(t.v))
      return fail(MATOPT_ERR_ALIGN, tag + ": pointer not 16-byte aligned");
    spans.push_back({(uintptr_t)t.p, (uintptr_t)t.p + (size_t)t.n * es, tag + " p"});
    spans.push_back({(uintptr_t)t.g, (uintptr_t)t.g + (size_t)t.n * es, tag + " g"});
    spans.push_back({(uintptr_t)t.m, (uintptr_t)t.m + (size_t)t.n * 4, tag + " m"});
    spans.push_back({(uintptr_t)t.v, (uintptr_t)t.v + (size_t)t.n * 4, tag + " v"});
    ptrs[i] = BindPtrs{{t.p, t.g, t.m, t.v}};
  }
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{PK_ADAMW, (uint64_t)dt, (uint64_t)dev, (uint64_t)count};
  for (int i = 0; i < count; ++i) key.push_back((uint64_t)vecs[i].n);
  std::shared_ptr<Plan> plan;
  st = get_plan(key, dev, s, [&](Plan& p) { return build_adamw_plan(p, vecs, count); }, plan);
  if (st != MATOPT_OK) return st;
  PlanUse use(*plan, s);
  if (use.error() != hipSuccess) return hip_fail("plan stream wait", use.error());
  VecDesc* slot = plan->dev<VecDesc>(plan->o_slot);
  if (!same_ptrs(ptrs, plan->slot_bound)) {
    plan->slot_bound.clear();
    if ((st = bind_descs(plan->dev<VecDesc>(plan->o_tmpl), slot, nullptr, BIND_VEC, ptrs, s)) !=
        MATOPT_OK)
      return st;
    plan->slot_bound = ptrs;
  }
  const double b1 = beta1, b2 = beta2;
  AdamwParams ap;
  ap.vecs = slot;
  ap.tasks = plan->dev<VecTask>(plan->rmnp[0].off);
  ap.b1 = b1;
  ap.omb1 = 1.0 - b1;
  ap.b2 = b2;
  ap.omb2 = 1.0 - b2;
  ap.step_size = (double)lr / (1.0 - std::pow(b1, (double)step));
  ap.inv_sqrt_bc2 = 1.0 / std::sqrt(1.0 - std::pow(b2, (double)step));
  ap.eps = eps;
  ap.wdl = (double)lr * (double)wd;
  hipError_t e = timed(9, s, [&] { return launch_adamw(dt, ap, plan->rmnp[0].n, s); });
  if (e != hipSuccess) return hip_fail("adamw launch", e);
  return MATOPT_OK;
}

matopt_status matopt_profile_enable(int32_t on) {
  if (on) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_clk.count(dev)) {
      unsigned long long* p = nullptr;
      const size_t bytes = 2 * MATOPT_PROFILE_CLASSES * sizeof(unsigned long long);
      e = hipMalloc(&p, bytes);
      if (e == hipSuccess) e = hipMemset(p, 0, bytes);
      if (e != hipSuccess) return hip_fail("profile clock buffer", e);
      g_prof_clk[dev] = p;
    }
  }
  g_prof.store(on != 0);
  return MATOPT_OK;
}

matopt_status matopt_profile_read_clock(double* mhz) {
  if (!mhz) return fail(MATOPT_ERR_NULL, "NULL output");
  for (int k = 0; k < MATOPT_PROFILE_CLASSES; ++k) mhz[k] = 0.0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  auto it = g_prof_clk.find(dev);
  if (it == g_prof_clk.end()) return MATOPT_OK;
  unsigned long long h[2 * MATOPT_PROFILE_CLASSES];
  const size_t bytes = sizeof(h);
  e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(h, it->second, bytes, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(it->second, 0, bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail("profile clock read", e);
  for (int k = 0; k < MATOPT_PROFILE_CLASSES; ++k)
    if (h[2 * k + 1]) mhz[k] = 100.0 * (double)h[2 * k] / (double)h[2 * k + 1];
  return MATOPT_OK;
}

matopt_status matopt_profile_read(double* ms, int64_t* launches) {
  if (!ms || !launches) return fail(MATOPT_ERR_NULL, "NULL output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : g_prof_pending) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail("profile event", e);
    g_prof_ms[r.cls] += t;
    g_prof_n[r.cls] += 1;
    g_ev_free.push_back(r.a);
    g_ev_free.push_back(r.b);
  }
  g_prof_pending.clear();
  for (int k = 0; k < MATOPT_PROFILE_CLASSES; ++k) {
    ms[k] = g_prof_ms[k];
    launches[k] = g_prof_n[k];
    g_prof_ms[k] = 0.0;
    g_prof_n[k] = 0;
  }
  return MATOPT_OK;
}

matopt_status matopt_mfma_probe(int32_t form, int32_t from_lds, const void* src, float* out,
                                int32_t iters, int32_t workgroups, uint64_t* clk,
                                void* stream) {
  if (!src || !out || !clk) return fail(MATOPT_ERR_NULL, "NULL src, out or clk");
  if (form != 16 && form != 32) return fail(MATOPT_ERR_PARAM, "form must be 16 or 32");
  if (iters < 2 || iters > (1 << 22) || (iters & 1))
    return fail(MATOPT_ERR_PARAM, "iters must be even, in [2, 2^22]");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(MATOPT_ERR_PARAM, "workgroups outside [1, 2^20]");
  if (((uintptr_t)src | (uintptr_t)out | (uintptr_t)clk) & 15)
    return fail(MATOPT_ERR_ALIGN, "src, out and clk must be 16-byte aligned");
  int dev = -1;
  matopt_status st;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  const hipError_t e = launch_mfma_probe(form == 16, from_lds != 0, src, out, iters, workgroups,
                                         (unsigned long long*)clk, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("mfma probe launch", e);
  return MATOPT_OK;
}

matopt_status matopt_counters(int64_t* out, int32_t n) {
  if (!out) return fail(MATOPT_ERR_NULL, "NULL output");
  if (n < 0 || n > MATOPT_COUNTERS) return fail(MATOPT_ERR_PARAM, "n outside [0, MATOPT_COUNTERS]");
  for (int k = 0; k < n; ++k) out[k] = g_counters[k].load(std::memory_order_relaxed);
  return MATOPT_OK;
}

}  // extern "C"
