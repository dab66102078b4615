// Host side of libmatopt: the C ABI declared in include/matopt.h.
//
// Each entry point validates its arguments synchronously, looks up (or builds
// once) a device-side plan for the exact list of shapes and pointers -- matrix
// descriptors plus the tile tables of every launch -- and enqueues the whole
// step on the caller's stream as a fixed sequence of grouped launches (every
// launch covers every matrix of the batch):
//
//   muon_step_batched        prep (momentum, norm partials, X0) -> finalize ->
//                            ns_steps x {Gram, polynomial, apply} (the last apply
//                            folds the update into W) | scale_out if ns_steps==0
//   ns_orthogonalize_batched same with no momentum; the last apply writes O
//   rmnp_step_batched        one fused row kernel launch per width class
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
int esize(int dt) { return dt == DT_BF16 ? 2 : 4; }
int gemm_tile(int dt) { return dt == DT_BF16 ? kTileBf16 : kTileF32; }

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
  g.prep_tc = cols_p / kPrepTile;
  return g;
}

struct Layout {
  std::vector<size_t> x0, x1, a, b;
  size_t partials = 0, xs = 0, total = 0;
  int n_prep = 0;
  std::vector<int> prep_off;
};

constexpr int64_t kMaxSide = 1 << 20;
constexpr int64_t kMaxElems = int64_t(1) << 32;

Layout layout(const std::vector<Geo>& geo, int dt) {
  Layout L;
  const size_t es = esize(dt);
  size_t off = 0;
  for (const Geo& g : geo) {
    const size_t xb = align256((size_t)g.mp * g.np * es);
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

// ---------------------------------------------------------------- plans
enum PlanKind {
  PK_MUON = 1, PK_NS = 2, PK_RMNP = 3, PK_COLCUT_PARTIAL = 4, PK_COLCUT_APPLY = 5, PK_ADAMW = 6
};

struct RmnpGroup {
  int wpr, nch, n;
  size_t off;  // byte offset of its task table in the plan buffer
};

// A GEMM stage's launch table and its length (the grid size of that stage:
// the three tables are packed separately and differ in length).
struct TileTable {
  const GemmTile* tiles = nullptr;
  int n = 0;
};

struct Plan {
  int device = -1;
  void* dbuf = nullptr;
  MatDesc* d_mats = nullptr;
  PrepTile* d_prep = nullptr;
  VecDesc* d_vecs = nullptr;   // AdamW plans
  TileTable gram, poly, apply;
  int count = 0, n_prep = 0;
  std::vector<RmnpGroup> rmnp;
  // Evicted plans are freed on their own device after it has drained (a queued
  // launch may still read the tables).  Plans alive at process exit are never
  // destroyed: the cache is a leaked singleton, so no HIP call runs during
  // static destruction.
  ~Plan() {
    if (!dbuf) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (device >= 0 && device != cur) (void)hipSetDevice(device);
    (void)hipDeviceSynchronize();
    (void)hipFree(dbuf);
    if (device >= 0 && device != cur) (void)hipSetDevice(cur);
  }
};

using PlanKey = std::vector<uint64_t>;
constexpr size_t kPlanCap = 64;
std::mutex g_plan_mu;
using PlanList = std::list<std::pair<PlanKey, std::shared_ptr<Plan>>>;
PlanList& g_plans = *new PlanList();  // front = most recent; never destroyed

std::shared_ptr<Plan> plan_lookup(const PlanKey& key) {
  for (auto it = g_plans.begin(); it != g_plans.end(); ++it)
    if (it->first == key) {
      g_plans.splice(g_plans.begin(), g_plans, it);
      return g_plans.front().second;
    }
  return nullptr;
}

void plan_insert(const PlanKey& key, std::shared_ptr<Plan> p) {
  g_plans.emplace_front(key, std::move(p));
  while (g_plans.size() > kPlanCap) g_plans.pop_back();
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
};

matopt_status upload(Plan& p, HostBuf& hb, hipStream_t s) {
  hipError_t e = hipMalloc(&p.dbuf, hb.bytes.size());
  if (e != hipSuccess) return fail(MATOPT_ERR_HIP, std::string("plan hipMalloc: ") + hipGetErrorString(e));
  e = hipMemcpyAsync(p.dbuf, hb.bytes.data(), hb.bytes.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MATOPT_ERR_HIP, std::string("plan upload: ") + hipGetErrorString(e));
  return MATOPT_OK;
}

template <typename T>
T* at(void* base, size_t off) {
  return (T*)((uint8_t*)base + off);
}

// Builds the descriptors and tile tables of a Newton-Schulz plan (muon / ns).
matopt_status build_ns_plan(Plan& P, int kind, int dt, const std::vector<Geo>& geo,
                            const std::vector<const void*>& wv, const std::vector<const void*>& gv,
                            const std::vector<const void*>& vv, const std::vector<const void*>& ov,
                            void* ws, hipStream_t s) {
  const int count = (int)geo.size();
  const Layout L = layout(geo, dt);
  const int tile = gemm_tile(dt);
  std::vector<MatDesc> mats(count);
  std::vector<PrepTile> prep;
  std::vector<TileUnit> u3, u4, u5;
  prep.reserve(L.n_prep);
  for (int i = 0; i < count; ++i) {
    const Geo& g = geo[i];
    MatDesc& d = mats[i];
    std::memset(&d, 0, sizeof(d));
    d.w = (void*)wv[i];
    d.g = gv[i];
    d.v = (void*)vv[i];
    d.o = (void*)ov[i];
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
    d.x[0] = at<void>(ws, L.x0[i]);
    d.x[1] = at<void>(ws, L.x1[i]);
    // X0 is the stored V; when V has X0's layout the first iteration reads it
    // in place and the prep kernel skips the copy
    d.x0_is_v = (dt == DT_BF16 && !g.transposed && g.rows == g.mp && g.cols == g.np) ? 1 : 0;
    d.x0in = d.x0_is_v ? vv[i] : d.x[0];
    d.a = at<void>(ws, L.a[i]);
    d.b = at<void>(ws, L.b[i]);
    d.xs = at<float>(ws, L.xs) + i;
    d.partials = at<float>(ws, L.partials) + L.prep_off[i];
    d.n_prep = g.prep_tr * g.prep_tc;
    int idx = 0;
    for (int tr = 0; tr < g.prep_tr; ++tr)
      for (int tc = 0; tc < g.prep_tc; ++tc) prep.push_back({i, tr, tc, idx++});
    const int tm = g.mp / tile, tn = g.np / tile;
    // diagonal tiles as the GEMM build treats them (bf16: 36 of their 64
    // blocks; the Gram's two per workgroup, in step with the matrix's other
    // tiles, which share their operand panels through L2)
    const int dm3 = dt == DT_BF16 ? gemm_bf16_diag_mode(0) : 0;
    const int dm4 = dt == DT_BF16 ? gemm_bf16_diag_mode(1) : 0;
    units_triangle(i, tm, g.np, u3, dm3 ? 9 : 16, dm3 == 2);
    units_triangle(i, tm, g.mp, u4, dm4 ? 9 : 16, dm4 == 2);
    units_full(i, tm, tn, g.mp, u5);
  }
  static_assert(sizeof(TileRef) == sizeof(GemmTile), "tile record layout");
  const std::vector<TileRef> k3 = xcd_schedule(u3), k4 = xcd_schedule(u4), k5 = xcd_schedule(u5);

  HostBuf hb;
  const size_t o_mats = hb.put(mats);
  const size_t o_prep = hb.put(prep);
  const size_t o_k3 = hb.put(k3);
  const size_t o_k4 = hb.put(k4);
  const size_t o_k5 = hb.put(k5);
  matopt_status st = upload(P, hb, s);
  if (st != MATOPT_OK) return st;
  P.d_mats = at<MatDesc>(P.dbuf, o_mats);
  P.d_prep = at<PrepTile>(P.dbuf, o_prep);
  P.gram = TileTable{at<GemmTile>(P.dbuf, o_k3), (int)k3.size()};
  P.poly = TileTable{at<GemmTile>(P.dbuf, o_k4), (int)k4.size()};
  P.apply = TileTable{at<GemmTile>(P.dbuf, o_k5), (int)k5.size()};
  P.count = count;
  P.n_prep = (int)prep.size();
  (void)kind;
  return MATOPT_OK;
}

matopt_status build_rmnp_plan(Plan& P, int dt, const matopt_mat* mats, int count, hipStream_t s) {
  const int E = 16 / esize(dt);
  std::vector<MatDesc> descs(count);
  std::map<std::pair<int, int>, std::vector<RmnpTask>> groups;
  for (int i = 0; i < count; ++i) {
    MatDesc& d = descs[i];
    std::memset(&d, 0, sizeof(d));
    d.w = mats[i].w;
    d.g = mats[i].g;
    d.v = mats[i].v;
    d.rows = mats[i].rows;
    d.cols = mats[i].cols;
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
  const size_t o_mats = hb.put(descs);
  for (auto& kv : groups) {
    RmnpGroup g;
    g.wpr = kv.first.first;
    g.nch = kv.first.second;
    g.n = (int)kv.second.size();
    g.off = hb.put(kv.second);
    P.rmnp.push_back(g);
  }
  matopt_status st = upload(P, hb, s);
  if (st != MATOPT_OK) return st;
  P.d_mats = at<MatDesc>(P.dbuf, o_mats);
  P.count = count;
  return MATOPT_OK;
}

matopt_status hip_fail(const char* what, hipError_t e) {
  return fail(MATOPT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Enqueue the Newton-Schulz pipeline of a plan.
matopt_status run_ns(const Plan& P, int dt, bool momentum, float mu, float lr, double wdl,
                     int ns_steps, float a, float b, float c, float eps, int out_kind,
                     int out_dt, hipStream_t s) {
  hipError_t e;
  PrepParams pp{P.d_mats, P.d_prep, mu, momentum ? 1 : 0};
  e = timed(0, s, [&] { return launch_prep(dt, pp, P.n_prep, s); });
  if (e != hipSuccess) return hip_fail("prep launch", e);
  FinalizeParams fp{P.d_mats, eps};
  e = timed(1, s, [&] { return launch_finalize(fp, P.count, s); });
  if (e != hipSuccess) return hip_fail("finalize launch", e);
  // every stage launches exactly its own table
  auto gemm = [&](GemmParams g, const TileTable& t) {
    g.tiles = t.tiles;
    return dt == DT_BF16 ? launch_gemm_bf16(g, t.n, s) : launch_gemm_f32(g, t.n, s);
  };
  for (int it = 0; it < ns_steps; ++it) {
    GemmParams g;
    std::memset(&g, 0, sizeof(g));
    g.mats = P.d_mats;
    g.cur = it & 1;
    g.first = it == 0 ? 1 : 0;
    g.out_dt = out_dt;
    g.a = a;
    g.b = b;
    g.c = c;
    g.lr = lr;
    g.wdl = wdl;
    g.stage = 0;
    g.out_kind = OUT_NEXT_X;
    e = timed(2, s, [&] { return gemm(g, P.gram); });
    if (e != hipSuccess) return hip_fail("gram launch", e);
    g.stage = 1;
    e = timed(3, s, [&] { return gemm(g, P.poly); });
    if (e != hipSuccess) return hip_fail("poly launch", e);
    g.stage = 2;
    g.out_kind = it == ns_steps - 1 ? out_kind : OUT_NEXT_X;
    e = timed(4, s, [&] { return gemm(g, P.apply); });
    if (e != hipSuccess) return hip_fail("apply launch", e);
  }
  if (ns_steps == 0) {
    ScaleOutParams sp{P.d_mats, P.d_prep, out_kind, out_dt, lr, wdl};
    e = timed(5, s, [&] { return launch_scale_out(dt, sp, P.n_prep, s); });
    if (e != hipSuccess) return hip_fail("scale_out launch", e);
  }
  return MATOPT_OK;
}

matopt_status check_common(int32_t count, int dt) {
  if (count < 0) return fail(MATOPT_ERR_PARAM, "count < 0");
  if (dt != DT_F32 && dt != DT_BF16) return fail(MATOPT_ERR_DTYPE, "dtype must be MATOPT_F32 or MATOPT_BF16");
  return MATOPT_OK;
}

matopt_status check_ns_params(int32_t ns_steps, float a, float b, float c, float eps) {
  if (ns_steps < 0 || ns_steps > 64) return fail(MATOPT_ERR_PARAM, "ns_steps outside [0, 64]");
  if (!finite(a) || !finite(b) || !finite(c)) return fail(MATOPT_ERR_PARAM, "non-finite Newton-Schulz coefficient");
  if (!finite(eps) || eps < 0.f) return fail(MATOPT_ERR_PARAM, "eps must be finite and >= 0");
  return MATOPT_OK;
}

// Column-cut RMNP plan: descriptors whose `partials` point into the caller's
// row-sum vector (matrix i starts at the sum of the rows before it) and one
// task per 4 rows.  full_cols (NULL: the slice's own width) sets the update
// scale from the whole matrix's shape.
matopt_status build_colcut_plan(Plan& P, int dt, const matopt_mat* mats, int count,
                                const float* rowsq, const int64_t* full_cols, hipStream_t s) {
  const int E = 16 / esize(dt);
  std::vector<MatDesc> descs(count);
  std::vector<RmnpTask> tasks;
  int64_t off = 0;
  for (int i = 0; i < count; ++i) {
    MatDesc& d = descs[i];
    std::memset(&d, 0, sizeof(d));
    d.w = mats[i].w;
    d.g = mats[i].g;
    d.v = mats[i].v;
    d.rows = mats[i].rows;
    d.cols = mats[i].cols;
    const int64_t fc = full_cols ? full_cols[i] : d.cols;
    d.upd_scale = (float)std::sqrt(std::max(1.0, (double)d.rows / (double)fc));
    d.vec_ok = d.cols % E == 0 ? 1 : 0;
    d.partials = const_cast<float*>(rowsq) + off;
    off += d.rows;
    for (int64_t r = 0; r < d.rows; r += 4) tasks.push_back({i, (int32_t)r});
  }
  HostBuf hb;
  const size_t o_mats = hb.put(descs);
  RmnpGroup g;
  g.wpr = 1;
  g.nch = 0;
  g.n = (int)tasks.size();
  g.off = hb.put(tasks);
  P.rmnp.push_back(g);
  matopt_status st = upload(P, hb, s);
  if (st != MATOPT_OK) return st;
  P.d_mats = at<MatDesc>(P.dbuf, o_mats);
  P.count = count;
  return MATOPT_OK;
}

// Shared by both column-cut halves: validation, plan lookup, one launch.
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
  }
  spans.push_back({(uintptr_t)rowsq, (uintptr_t)rowsq + (size_t)total_rows * 4, "rowsq"});
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{(uint64_t)(apply ? PK_COLCUT_APPLY : PK_COLCUT_PARTIAL), (uint64_t)dt, (uint64_t)dev,
              (uint64_t)count, (uint64_t)(uintptr_t)rowsq};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)mats[i].rows);
    key.push_back((uint64_t)mats[i].cols);
    key.push_back((uint64_t)(uintptr_t)(apply ? mats[i].w : mats[i].g));
    key.push_back((uint64_t)(uintptr_t)mats[i].v);
    key.push_back((uint64_t)(apply && full_cols ? full_cols[i] : mats[i].cols));
  }
  std::shared_ptr<Plan> plan;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    plan = plan_lookup(key);
    if (!plan) {
      plan = std::make_shared<Plan>();
      plan->device = dev;
      if ((st = build_colcut_plan(*plan, dt, mats, count, rowsq, apply ? full_cols : nullptr, s)) !=
          MATOPT_OK)
        return st;
      plan_insert(key, plan);
    }
  }
  const RmnpGroup& g = plan->rmnp[0];
  ColcutParams cp{plan->d_mats, at<RmnpTask>(plan->dbuf, g.off), mu, lr, eps};
  hipError_t e = timed(apply ? 8 : 7, s, [&] { return launch_colcut(dt, apply, cp, g.n, s); });
  if (e != hipSuccess) return hip_fail(apply ? "colcut apply launch" : "colcut partial launch", e);
  return MATOPT_OK;
}

// AdamW plan: one descriptor per tensor and one task per kAdamwTask elements.
matopt_status build_adamw_plan(Plan& P, const matopt_vec* vecs, int count, hipStream_t s) {
  std::vector<VecDesc> descs(count);
  std::vector<VecTask> tasks;
  for (int i = 0; i < count; ++i) {
    descs[i] = VecDesc{vecs[i].p, vecs[i].g, vecs[i].m, vecs[i].v, vecs[i].n};
    for (int64_t e = 0; e < vecs[i].n; e += kAdamwTask) tasks.push_back({i, 0, e});
  }
  HostBuf hb;
  const size_t o_vecs = hb.put(descs);
  RmnpGroup g;
  g.wpr = 0;
  g.nch = 0;
  g.n = (int)tasks.size();
  g.off = hb.put(tasks);
  P.rmnp.push_back(g);
  matopt_status st = upload(P, hb, s);
  if (st != MATOPT_OK) return st;
  P.d_vecs = at<VecDesc>(P.dbuf, o_vecs);
  P.count = count;
  return MATOPT_OK;
}

}  // namespace

// ==================================================================== C ABI
extern "C" {

int32_t matopt_version(void) { return 10000; }

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
  if (dt != MATOPT_F32 && dt != MATOPT_BF16) return 0;
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
  matopt_status st = check_common(count, dt);
  if (st != MATOPT_OK) return st;
  if (count == 0) return MATOPT_OK;
  if (!mats) return fail(MATOPT_ERR_NULL, "mats is NULL");
  if (!finite(mu) || !finite(lr)) return fail(MATOPT_ERR_PARAM, "non-finite mu or lr");
  if (!finite(wd)) return fail(MATOPT_ERR_PARAM, "non-finite weight decay");
  if ((st = check_ns_params(ns_steps, a, b, c, eps)) != MATOPT_OK) return st;
  std::vector<Geo> geo;
  std::vector<Span> spans;
  std::vector<const void*> wv, gv, vv, ov;
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
    wv.push_back(m.w);
    gv.push_back(m.g);
    vv.push_back(m.v);
    ov.push_back(nullptr);
  }
  const size_t need = layout(geo, dt).total;
  if (!workspace || workspace_bytes < need)
    return fail(MATOPT_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                          std::to_string(workspace ? workspace_bytes : 0));
  if (((uintptr_t)workspace & 255) != 0) return fail(MATOPT_ERR_ALIGN, "workspace not 256-byte aligned");
  spans.push_back({(uintptr_t)workspace, (uintptr_t)workspace + need, "workspace"});
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;

  PlanKey key{PK_MUON, (uint64_t)dt, (uint64_t)dev, (uint64_t)(uintptr_t)workspace, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)mats[i].rows);
    key.push_back((uint64_t)mats[i].cols);
    key.push_back((uint64_t)(uintptr_t)mats[i].w);
    key.push_back((uint64_t)(uintptr_t)mats[i].g);
    key.push_back((uint64_t)(uintptr_t)mats[i].v);
  }
  std::shared_ptr<Plan> plan;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    plan = plan_lookup(key);
    if (!plan) {
      plan = std::make_shared<Plan>();
      plan->device = dev;
      if ((st = build_ns_plan(*plan, PK_MUON, dt, geo, wv, gv, vv, ov, workspace, s)) != MATOPT_OK) return st;
      plan_insert(key, plan);
    }
  }
  const double wdl = (double)lr * (double)wd;   // exact: a product of two floats
  return run_ns(*plan, dt, true, mu, lr, wdl, ns_steps, a, b, c, eps, OUT_W_UPDATE, dt, s);
}

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
  matopt_status st = check_common(count, in_dt);
  if (st != MATOPT_OK) return st;
  if (out_dt != MATOPT_F32 && out_dt != MATOPT_BF16) return fail(MATOPT_ERR_DTYPE, "invalid out_dt");
  if (count == 0) return MATOPT_OK;
  if (!x || !o || !rows || !cols) return fail(MATOPT_ERR_NULL, "NULL argument array");
  if ((st = check_ns_params(ns_steps, a, b, c, eps)) != MATOPT_OK) return st;
  std::vector<Geo> geo;
  std::vector<Span> spans;
  std::vector<const void*> wv, gv, vv, ov;
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
    wv.push_back(nullptr);
    gv.push_back(nullptr);
    vv.push_back(x[i]);
    ov.push_back(o[i]);
  }
  const size_t need = layout(geo, in_dt).total;
  if (!workspace || workspace_bytes < need)
    return fail(MATOPT_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                          std::to_string(workspace ? workspace_bytes : 0));
  if (((uintptr_t)workspace & 255) != 0) return fail(MATOPT_ERR_ALIGN, "workspace not 256-byte aligned");
  spans.push_back({(uintptr_t)workspace, (uintptr_t)workspace + need, "workspace"});
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;

  PlanKey key{PK_NS, (uint64_t)in_dt, (uint64_t)dev, (uint64_t)(uintptr_t)workspace, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)rows[i]);
    key.push_back((uint64_t)cols[i]);
    key.push_back((uint64_t)(uintptr_t)x[i]);
    key.push_back((uint64_t)(uintptr_t)o[i]);
  }
  std::shared_ptr<Plan> plan;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    plan = plan_lookup(key);
    if (!plan) {
      plan = std::make_shared<Plan>();
      plan->device = dev;
      if ((st = build_ns_plan(*plan, PK_NS, in_dt, geo, wv, gv, vv, ov, workspace, s)) != MATOPT_OK) return st;
      plan_insert(key, plan);
    }
  }
  return run_ns(*plan, in_dt, false, 0.f, 0.f, 0.0, ns_steps, a, b, c, eps, OUT_O, out_dt, s);
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
  }
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{PK_RMNP, (uint64_t)dt, (uint64_t)dev, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)mats[i].rows);
    key.push_back((uint64_t)mats[i].cols);
    key.push_back((uint64_t)(uintptr_t)mats[i].w);
    key.push_back((uint64_t)(uintptr_t)mats[i].g);
    key.push_back((uint64_t)(uintptr_t)mats[i].v);
  }
  std::shared_ptr<Plan> plan;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    plan = plan_lookup(key);
    if (!plan) {
      plan = std::make_shared<Plan>();
      plan->device = dev;
      if ((st = build_rmnp_plan(*plan, dt, mats, count, s)) != MATOPT_OK) return st;
      plan_insert(key, plan);
    }
  }
  RmnpParams rp{plan->d_mats, nullptr, mu, lr, eps};
  for (const RmnpGroup& g : plan->rmnp) {
    rp.tasks = at<RmnpTask>(plan->dbuf, g.off);
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
  }
  if ((st = check_overlap(spans)) != MATOPT_OK) return st;
  int dev;
  if ((st = check_device(&dev)) != MATOPT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  PlanKey key{PK_ADAMW, (uint64_t)dt, (uint64_t)dev, (uint64_t)count};
  for (int i = 0; i < count; ++i) {
    key.push_back((uint64_t)vecs[i].n);
    key.push_back((uint64_t)(uintptr_t)vecs[i].p);
    key.push_back((uint64_t)(uintptr_t)vecs[i].g);
    key.push_back((uint64_t)(uintptr_t)vecs[i].m);
    key.push_back((uint64_t)(uintptr_t)vecs[i].v);
  }
  std::shared_ptr<Plan> plan;
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    plan = plan_lookup(key);
    if (!plan) {
      plan = std::make_shared<Plan>();
      plan->device = dev;
      if ((st = build_adamw_plan(*plan, vecs, count, s)) != MATOPT_OK) return st;
      plan_insert(key, plan);
    }
  }
  const double b1 = beta1, b2 = beta2;
  AdamwParams ap;
  ap.vecs = plan->d_vecs;
  ap.tasks = at<VecTask>(plan->dbuf, plan->rmnp[0].off);
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
  g_prof.store(on != 0);
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

}  // extern "C"
