// Host runtime behind the C ABI of include/matrix_roots.h: argument
// validation (all-or-nothing, before anything is enqueued), workspace layout,
// work lists and launch order.  No device allocation, no descriptor copies:
// per-problem tables travel in kernel arguments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "cans.hpp"
#include "launch.hpp"
#include "peaks.hpp"
#include "polar.hpp"
#include "step.hpp"
#include "schedule.hpp"

using namespace mr;

namespace {

thread_local std::string g_err;

mr_status fail(mr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

mr_status hip_fail(hipError_t e, const char* where) {
  return fail(MR_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = 65536;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range of a rows x cols row-major matrix with leading dimension ld.
struct Range {
  uintptr_t lo, hi;
};
Range range_of(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t es) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * (int64_t)es)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
// Byte range of a symmetric d x d matrix, full (leading dimension ld) or packed.
Range sym_range_of(const void* p, int64_t d, int64_t ld, size_t es, bool packed) {
  return packed ? range_of(p, 1, d * (d + 1) / 2, 0, es) : range_of(p, d, d, ld, es);
}
// All-or-nothing alias check over a whole batch: no byte range a call writes
// may overlap another one it writes or one it reads, within a problem or
// across problems (inputs may share memory with each other).
struct AliasSet {
  struct Tagged {
    Range r;
    int problem;
    const char* name;
  };
  std::vector<Tagged> outs, ins;
  void out(Range r, int i, const char* name) { outs.push_back({r, i, name}); }
  void in(Range r, int i, const char* name) { ins.push_back({r, i, name}); }
  mr_status check() {
    std::sort(outs.begin(), outs.end(), [](const Tagged& a, const Tagged& b) { return a.r.lo < b.r.lo; });
    for (size_t k = 1; k < outs.size(); ++k)
      if (outs[k].r.lo < outs[k - 1].r.hi)
        return fail(MR_ERR_ALIAS, "problem %d: %s overlaps problem %d's %s", outs[k].problem, outs[k].name,
                    outs[k - 1].problem, outs[k - 1].name);
    // the outputs are now disjoint and sorted, so the last one starting before
    // an input ends is the only one that can overlap it
    for (const Tagged& x : ins) {
      auto it = std::lower_bound(outs.begin(), outs.end(), x.r.hi,
                                 [](const Tagged& a, uintptr_t v) { return a.r.lo < v; });
      if (it != outs.begin() && std::prev(it)->r.hi > x.r.lo)
        return fail(MR_ERR_ALIAS, "problem %d: %s overlaps problem %d's %s", std::prev(it)->problem,
                    std::prev(it)->name, x.problem, x.name);
    }
    return MR_OK;
  }
};

// Base dtype and storage flag of an mr_dtype argument.
mr_dtype base_dtype(mr_dtype dt) { return dt & ~MR_PACKED; }
bool is_packed(mr_dtype dt) { return (dt & MR_PACKED) != 0; }
bool valid_dtype(mr_dtype dt) { return (dt & ~(MR_PACKED | 1)) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = getenv("MR_DEBUG_SYNC");
    return e && e[0] == '1';
  }();
  return on;
}

// Check a launch; in debug mode also wait for it and report faults there.
mr_status check_launch(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return MR_OK;
}

int tiles(int64_t d, int t) { return (int)((d + t - 1) / t); }
// workgroups of the upper tile pairs (upper_pair) of a d x d matrix
int upper_tiles(int64_t d, int t) {
  const int T = tiles(d, t);
  return T * (T + 1) / 2;
}

// ------------------------------------------------------------ tracing
enum TraceClass {
  kTrSyrk, kTrJacobi, kTrStats, kTrBound, kTrInit, kTrNewton64, kTrNewton32, kTrConvert,
  kTrFinalize, kTrInfo, kTrNewtonX3, kTrCansBound, kTrCansInit, kTrCansP, kTrCansYZ, kTrCansFinal, kTrCansInfo,
  kTrPolarStats, kTrPolarBound, kTrPolarInit, kTrPolarA, kTrPolarX, kTrPolarFinal, kTrPolarInfo,
  kTrMomentum, kTrHyperReduce, kTrHyperUpdate, kTrApplyX3, kTrApplySplit, kTrSlice, kTrNewtonI8, kTrMoment, kTrCount
};
const char* const kTraceNames[kTrCount] = {"syrk_ema", "jacobi", "root_stats", "root_bound",
                                           "root_init", "newton_f64", "newton_f32", "newton_convert",
                                           "root_finalize", "root_info", "newton_x3", "cans_bound",
                                           "cans_init", "cans_p", "cans_yz", "cans_finalize", "cans_info",
                                           "polar_stats", "polar_bound", "polar_init", "polar_gram",
                                           "polar_update", "polar_finalize", "polar_info", "momentum",
                                           "hyperball_reduce", "hyperball_update", "apply_x3", "apply_split",
                                           "newton_slice", "newton_i8", "root_moment"};
struct TraceEntry {
  int cls;
  hipEvent_t a, b;
};
struct Trace {
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<TraceEntry> log;
  std::mutex mu;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Trace g_trace;

// Launch through `fn`; in trace mode bracket it with events on its stream.
template <class F>
mr_status traced(int cls, bool nonempty, hipStream_t s, F&& fn, const char* what) {
  if (!g_trace.on || !nonempty) return check_launch(fn(), s, what);
  std::lock_guard<std::mutex> lk(g_trace.mu);
  hipEvent_t a = g_trace.get(), b = g_trace.get();
  if (!a || !b) return fail(MR_ERR_HIP, "%s: hipEventCreate failed", what);
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = fn();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  g_trace.log.push_back({cls, a, b});
  return check_launch(e, s, what);
}

// ------------------------------------------------------------ root layout
struct RootPlan {
  // slot order: Newton matrices grouped by d (ascending), then Jacobi
  std::vector<int> slot_problem;
  int n_newton = 0;
  struct Cls {
    int64_t d;
    int first_slot, count;
    size_t region_off, matrix_bytes;
  };
  std::vector<Cls> classes;
  size_t state_off = 0, partial_off = 0, sched_off = 0, jac_desc_off = 0;
  int64_t partial_stride = 0;
  std::vector<size_t> jac_w_off;  // per Jacobi slot (index slot - n_newton); 0 when W stays in LDS
  int jac_first[kJacobiClasses] = {0, 0, 0, 0}, jac_count[kJacobiClasses] = {0, 0, 0, 0};  // slot ranges
  size_t total = 0;
};

// Sweep cap of the Jacobi route (mr_set_jacobi_max_sweeps).
std::atomic<int32_t> g_jacobi_max_sweeps{kJacobiDefaultSweeps};

// Default Newton path: X in split-fp16 storage from the first step, the
// float64 steps' products on int8 digit planes from kI8MinD.
bool split_path(int32_t method) { return method != MR_NEWTON_F64 && method != MR_NEWTON_F32; }

bool use_jacobi(int64_t d, int32_t method) {
  return method == MR_JACOBI || (method == MR_AUTO && d <= kJacobiAutoMaxD);
}

RootPlan plan_root(const mr_root_problem* p, int32_t count, int32_t method) {
  RootPlan P;
  std::map<int64_t, std::vector<int>> by_d;
  std::vector<int> jac;
  for (int i = 0; i < count; ++i) {
    if (use_jacobi(p[i].d, method))
      jac.push_back(i);
    else
      by_d[p[i].d].push_back(i);
  }
  int64_t dmax_newton = 0;
  for (auto& kv : by_d) {
    RootPlan::Cls c;
    c.d = kv.first;
    c.first_slot = (int)P.slot_problem.size();
    c.count = (int)kv.second.size();
    // five float64 slots; the split-storage path adds what of the digit
    // planes of its float64 steps does not fit in them (d >= kI8MinD)
    c.matrix_bytes =
        (size_t)oz_f64_bytes(c.d) + (split_path(method) && c.d >= kI8MinD ? (size_t)oz_layout(c.d).extra : 0);
    for (int i : kv.second) P.slot_problem.push_back(i);
    P.classes.push_back(c);
    dmax_newton = std::max(dmax_newton, c.d);
  }
  P.n_newton = (int)P.slot_problem.size();
  // Jacobi slots grouped by size class (each class is one launch)
  std::stable_sort(jac.begin(), jac.end(), [&](int x, int y) { return jacobi_class_of(p[x].d) < jacobi_class_of(p[y].d); });
  for (size_t k = 0; k < jac.size(); ++k) {
    const int c = jacobi_class_of(p[jac[k]].d);
    if (P.jac_count[c] == 0) P.jac_first[c] = P.n_newton + (int)k;
    ++P.jac_count[c];
    P.slot_problem.push_back(jac[k]);
  }

  size_t off = 0;
  P.state_off = off;
  off = align256(off + sizeof(RootState) * (size_t)std::max(count, 1));
  P.partial_stride = std::max<int64_t>(3 * ((dmax_newton + kStatsRows - 1) / kStatsRows),
                                       (dmax_newton + kFinalRows - 1) / kFinalRows);
  // the moment bounds: |B/c|_F^2 and one sum per upper tile of H H and of P16 P16
  if (dmax_newton >= kMomentMinD)
    P.partial_stride = std::max<int64_t>(P.partial_stride, 2 + 2 * (int64_t)moment_tiles((int)dmax_newton));
  P.partial_stride = std::max<int64_t>(P.partial_stride, 1);
  P.partial_off = off;
  off = align256(off + sizeof(double) * (size_t)P.partial_stride * (size_t)std::max(P.n_newton, 1));
  P.sched_off = off;
  off = align256(off + sizeof(double) * kMaxNewtonIters * (size_t)std::max(P.n_newton, 1));
  P.jac_desc_off = off;
  off = align256(off + sizeof(JacobiDesc) * jac.size());
  for (size_t k = 0; k < jac.size(); ++k) {
    const int64_t d = p[jac[k]].d;
    if (d + (d & 1) <= kJacobiLdsW) {
      P.jac_w_off.push_back(0);
      continue;
    }
    P.jac_w_off.push_back(off);
    off = align256(off + sizeof(double) * (size_t)d * (size_t)d);
  }
  for (auto& c : P.classes) {
    c.region_off = off;
    off += c.matrix_bytes * (size_t)c.count;
  }
  P.total = off;
  return P;
}

}  // namespace

extern "C" {

int32_t mr_abi_version(void) { return MR_ABI_VERSION; }

int32_t mr_set_jacobi_max_sweeps(int32_t sweeps) {
  if (sweeps < 1 || sweeps > kJacobiMaxSweeps) return -1;
  return g_jacobi_max_sweeps.exchange(sweeps);
}

const char* mr_last_error_message(void) { return g_err.c_str(); }

const char* mr_status_string(mr_status s) {
  switch (s) {
    case MR_OK: return "MR_OK";
    case MR_ERR_NULL: return "MR_ERR_NULL: a required pointer is NULL";
    case MR_ERR_SHAPE: return "MR_ERR_SHAPE: invalid or inconsistent size";
    case MR_ERR_STRIDE: return "MR_ERR_STRIDE: leading dimension smaller than the column count";
    case MR_ERR_PARAM: return "MR_ERR_PARAM: scalar parameter or enum out of range";
    case MR_ERR_WORKSPACE: return "MR_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MR_ERR_HIP: return "MR_ERR_HIP: HIP runtime error";
    case MR_ERR_UNSUPPORTED: return "MR_ERR_UNSUPPORTED: request not implemented";
    case MR_ERR_ALIAS: return "MR_ERR_ALIAS: output overlaps an input";
    default: return "unknown mr_status";
  }
}

int32_t mr_trace_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_trace.mu);
  const int32_t prev = g_trace.on ? 1 : 0;
  g_trace.on = on != 0;
  return prev;
}

int32_t mr_trace_collect(mr_trace_record* out, int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_trace.mu);
  double ms[kTrCount] = {0};
  int64_t n[kTrCount] = {0};
  for (const TraceEntry& t : g_trace.log) {
    float e = 0.f;
    if (hipEventSynchronize(t.b) == hipSuccess && hipEventElapsedTime(&e, t.a, t.b) == hipSuccess) {
      ms[t.cls] += e;
      n[t.cls] += 1;
    }
    g_trace.pool.push_back(t.a);
    g_trace.pool.push_back(t.b);
  }
  g_trace.log.clear();
  int32_t k = 0;
  for (int c = 0; c < kTrCount; ++c) {
    if (n[c] == 0) continue;
    if (out && k < capacity) {
      memset(out[k].name, 0, sizeof out[k].name);
      strncpy(out[k].name, kTraceNames[c], sizeof out[k].name - 1);
      out[k].launches = n[c];
      out[k].total_ms = ms[c];
    }
    ++k;
  }
  return std::min(k, capacity);
}

int32_t mr_newton_schedule(double m0, double* scales, int32_t capacity, int32_t* fp64_steps,
                           int32_t* final_degree) {
  if (!(m0 > 0.0 && m0 <= 1.0 / kBoundSafety) || capacity < 0) return -1;
  double tmp[kMaxNewtonIters];
  int K = 0, j = 0, fin = 1;
  newton_scaled_schedule(m0, 1.0 / kBoundSafety, kNewtonTol, kSwitchM, kMaxNewtonIters, tmp, &K, &j, true, &fin);
  if (scales)
    for (int i = 0; i < K && i < capacity; ++i) scales[i] = tmp[i];
  if (fp64_steps) *fp64_steps = j;
  if (final_degree) *final_degree = fin;
  return K;
}

mr_status mr_measure_peaks(mr_peak_info* out, void* hip_stream) {
  if (!out) return fail(MR_ERR_NULL, "out is NULL");
  memset(out, 0, sizeof *out);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  out->cu_count = prop.multiProcessorCount;
  out->clock_khz = prop.clockRate;
  for (int k = 0; k < kPeakKinds; ++k)
    out->prop_tflops[k] = prop.multiProcessorCount * (prop.clockRate * 1e3) * kMfmaFlopsPerClockCU[k] / 1e12;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipEvent_t a = nullptr, b = nullptr;
  if ((e = hipEventCreate(&a)) != hipSuccess) return hip_fail(e, "hipEventCreate");
  if ((e = hipEventCreate(&b)) != hipSuccess) {
    (void)hipEventDestroy(a);
    return hip_fail(e, "hipEventCreate");
  }
  // eight workgroups (two waves per SIMD) per CU, about 5 ms per kind at the
  // vendor peak; the first launch of each kind warms the clock up
  const int blocks = 8 * std::max(1, prop.multiProcessorCount);
  const int iters[kPeakKinds] = {3000, 1500, 6000, 6000};
  mr_status st = MR_OK;
  for (int r = 0; r < 2; ++r)
    for (int k = 0; k < kPeakKinds && st == MR_OK; ++k) {
      double flops = 0.0;
      float ms = 0.f;
      e = launch_peak_loop(k, blocks, iters[k], r == 1, &flops, s);
      if (e == hipSuccess) e = hipEventRecord(a, s);
      if (e == hipSuccess) e = launch_peak_loop(k, blocks, iters[k], r == 1, &flops, s);
      if (e == hipSuccess) e = hipEventRecord(b, s);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      if (e != hipSuccess)
        st = hip_fail(e, "peak loop");
      else
        (r == 0 ? out->measured_tflops : out->measured_random_tflops)[k] =
            ms > 0.f ? flops / (ms * 1e-3) / 1e12 : 0.0;
    }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return st;
}

int32_t mr_newton_iterations(int32_t p, double m0, double tol) {
  if (!(p == 2 || p == 4) || !(m0 > 0.0 && m0 <= 1.0) || !(tol > 0.0 && tol < 1.0)) return -1;
  double m = m0;
  int k = 0;
  while (1.0 - m > tol && k < 100000) {
    m = newton_scalar_step(p, m);
    ++k;
  }
  return k;
}

// ======================================================== gram_ema_update
static mr_status validate_gram(const mr_gram_problem* p, int32_t count, mr_dtype dt, double beta, uint32_t sides) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!valid_dtype(dt))
    return fail(MR_ERR_PARAM, "state_dtype %d is not MR_F32 or MR_F64 (optionally | MR_PACKED)", dt);
  const bool packed = is_packed(dt);
  if (!(beta >= 0.0 && beta < 1.0)) return fail(MR_ERR_PARAM, "beta %g not in [0, 1)", beta);
  if (sides == 0 || (sides & ~(uint32_t)(MR_LEFT | MR_RIGHT)))
    return fail(MR_ERR_PARAM, "sides 0x%x must be a non-empty subset of MR_LEFT|MR_RIGHT", sides);
  const size_t es = base_dtype(dt) == MR_F64 ? 8 : 4;
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    const mr_gram_problem& q = p[i];
    if (q.m < 1 || q.n < 1 || q.m > kMaxDim || q.n > kMaxDim)
      return fail(MR_ERR_SHAPE, "problem %d: m=%lld n=%lld outside [1, %lld]", i, (long long)q.m, (long long)q.n,
                  (long long)kMaxDim);
    if (!q.G) return fail(MR_ERR_NULL, "problem %d: G is NULL", i);
    if (q.ldg < q.n) return fail(MR_ERR_STRIDE, "problem %d: ldg %lld < n %lld", i, (long long)q.ldg, (long long)q.n);
    if (!aligned(q.G, 4)) return fail(MR_ERR_PARAM, "problem %d: G not 4-byte aligned", i);
    const Range rg = range_of(q.G, q.m, q.n, q.ldg, 4);
    Range rl{0, 0}, rr{0, 0};
    if (sides & MR_LEFT) {
      if (!q.L) return fail(MR_ERR_NULL, "problem %d: L is NULL", i);
      if (!packed && q.ldl < q.m)
        return fail(MR_ERR_STRIDE, "problem %d: ldl %lld < m %lld", i, (long long)q.ldl, (long long)q.m);
      if (!aligned(q.L, es)) return fail(MR_ERR_PARAM, "problem %d: L misaligned for its dtype", i);
      rl = sym_range_of(q.L, q.m, q.ldl, es, packed);
      if (overlap(rl, rg)) return fail(MR_ERR_ALIAS, "problem %d: L overlaps G", i);
    }
    if (sides & MR_RIGHT) {
      if (!q.R) return fail(MR_ERR_NULL, "problem %d: R is NULL", i);
      if (!packed && q.ldr < q.n)
        return fail(MR_ERR_STRIDE, "problem %d: ldr %lld < n %lld", i, (long long)q.ldr, (long long)q.n);
      if (!aligned(q.R, es)) return fail(MR_ERR_PARAM, "problem %d: R misaligned for its dtype", i);
      rr = sym_range_of(q.R, q.n, q.ldr, es, packed);
      if (overlap(rr, rg)) return fail(MR_ERR_ALIAS, "problem %d: R overlaps G", i);
    }
    if ((sides & MR_LEFT) && (sides & MR_RIGHT) && overlap(rl, rr))
      return fail(MR_ERR_ALIAS, "problem %d: L overlaps R", i);
    al.in(rg, i, "G");
    if (sides & MR_LEFT) al.out(rl, i, "L");
    if (sides & MR_RIGHT) al.out(rr, i, "R");
  }
  return al.check();
}

size_t gram_ema_update_workspace(const mr_gram_problem*, int32_t, mr_dtype, uint32_t) { return 0; }

mr_status gram_ema_update(const mr_gram_problem* p, int32_t count, mr_dtype dt, double beta, uint32_t sides, void* ws,
                          size_t ws_bytes, void* hip_stream) {
  (void)ws;
  (void)ws_bytes;
  mr_status st = validate_gram(p, count, dt, beta, sides);
  if (st != MR_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  for (int side = 0; side < 2; ++side) {
    const bool right = side == 1;
    if (!(sides & (right ? MR_RIGHT : MR_LEFT))) continue;
    for (int vecpass = 0; vecpass < 2; ++vecpass) {
      const int vec = vecpass == 0 ? 4 : 1;
      SyrkBatch b;
      memset(&b, 0, sizeof b);
      b.alpha = 1.0 - beta;
      b.beta = beta;
      b.packed = is_packed(dt) ? 1 : 0;
      auto flush = [&]() -> mr_status {
        if (b.njobs == 0) return MR_OK;
        mr_status r = traced(kTrSyrk, b.total_blocks > 0, s,
                             [&] { return launch_syrk_ema(b, right, base_dtype(dt) == MR_F64, vec, s); },
                             "gram_ema_update launch");
        b.njobs = 0;
        b.total_blocks = 0;
        return r;
      };
      // Largest Grams first in each launch: their long tiles start early and
      // the short tiles of the small Grams fill the launch's tail.
      std::vector<int> order(count);
      for (int i = 0; i < count; ++i) order[i] = i;
      std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
        const int64_t dx = right ? p[x].n : p[x].m, dy = right ? p[y].n : p[y].m;
        const int64_t kx = right ? p[x].m : p[x].n, ky = right ? p[y].m : p[y].n;
        return dx * dx * kx > dy * dy * ky;
      });
      for (const int i : order) {
        const mr_gram_problem& q = p[i];
        const int64_t d = right ? q.n : q.m;
        const int64_t K = right ? q.m : q.n;
        // float4 loads: along columns of G (k for the left Gram, i for the right one)
        const bool v4 = (q.n % 4 == 0) && (q.ldg % 4 == 0) && aligned(q.G, 16);
        if ((vec == 4) != v4) continue;
        SyrkJob& J = b.job[b.njobs];
        J.G = q.G;
        J.ldg = q.ldg;
        J.S = right ? q.R : q.L;
        J.lds = right ? q.ldr : q.ldl;
        J.d = (int32_t)d;
        J.K = (int32_t)K;
        J.T = tiles(d, 128);
        J.block_begin = b.total_blocks;
        b.total_blocks += round8(J.T * (J.T + 1) / 2);
        ++b.njobs;
        if (b.njobs == kMaxSyrkJobs && (st = flush()) != MR_OK) return st;
      }
      if ((st = flush()) != MR_OK) return st;
    }
  }
  return MR_OK;
}

// ===================================================== precondition_apply
static mr_status validate_apply(const mr_apply_problem* p, int32_t count, float alpha) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!std::isfinite(alpha)) return fail(MR_ERR_PARAM, "alpha is not finite");
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    const mr_apply_problem& q = p[i];
    if (q.m < 1 || q.n < 1 || q.m > kMaxDim || q.n > kMaxDim)
      return fail(MR_ERR_SHAPE, "problem %d: m=%lld n=%lld outside [1, %lld]", i, (long long)q.m, (long long)q.n,
                  (long long)kMaxDim);
    if (!q.XL || !q.G || !q.XR || !q.U) return fail(MR_ERR_NULL, "problem %d: NULL matrix pointer", i);
    if (q.ldxl < q.m || q.ldg < q.n || q.ldxr < q.n || q.ldu < q.n)
      return fail(MR_ERR_STRIDE, "problem %d: a leading dimension is smaller than its column count", i);
    if (!aligned(q.XL, 4) || !aligned(q.G, 4) || !aligned(q.XR, 4) || !aligned(q.U, 4))
      return fail(MR_ERR_PARAM, "problem %d: a matrix is not 4-byte aligned", i);
    const Range ru = range_of(q.U, q.m, q.n, q.ldu, 4);
    if (overlap(ru, range_of(q.XL, q.m, q.m, q.ldxl, 4)) || overlap(ru, range_of(q.G, q.m, q.n, q.ldg, 4)) ||
        overlap(ru, range_of(q.XR, q.n, q.n, q.ldxr, 4)))
      return fail(MR_ERR_ALIAS, "problem %d: U overlaps XL, G or XR", i);
    al.out(ru, i, "U");
    al.in(range_of(q.XL, q.m, q.m, q.ldxl, 4), i, "XL");
    al.in(range_of(q.G, q.m, q.n, q.ldg, 4), i, "G");
    al.in(range_of(q.XR, q.n, q.n, q.ldxr, 4), i, "XR");
  }
  return al.check();
}

// Split apply workspace of one problem: split copies (4 bytes per element)
// of XR (n x n32), G (m x n32), XL (m x m32) and W^T (n x m32), and W^T in
// float32 (n x m); each 256-aligned.  After all problems: the largest
// magnitudes of every problem's XR, G, XL and W^T (4 words each).
struct ApplySplitLayout {
  size_t xr, g, xl, wt, wt32, end;
  int64_t n32, m32;
};
static ApplySplitLayout apply_split_layout(const mr_apply_problem& q, size_t off) {
  ApplySplitLayout L;
  L.n32 = (q.n + 31) / 32 * 32;
  L.m32 = (q.m + 31) / 32 * 32;
  L.xr = off;
  L.g = L.xr + align256((size_t)q.n * L.n32 * 4);
  L.xl = L.g + align256((size_t)q.m * L.n32 * 4);
  L.wt = L.xl + align256((size_t)q.m * L.m32 * 4);
  L.wt32 = L.wt + align256((size_t)q.n * L.m32 * 4);
  L.end = L.wt32 + align256((size_t)q.n * q.m * 4);
  return L;
}

size_t precondition_apply_workspace(const mr_apply_problem* p, int32_t count) {
  if (!p || count <= 0) return 0;
  size_t tot = 0;
  for (int i = 0; i < count; ++i) {
    if (p[i].m <= 0 || p[i].n <= 0) continue;
    tot = apply_split_layout(p[i], tot).end;
  }
  tot += align256((size_t)count * 4 * sizeof(uint32_t));
  return tot;
}

// U = alpha XL G XR with split operands: maxima and split copies of XR^T, G
// and XL; W^T = XR^T G^T = (G XR)^T (float32); its maxima and split copy;
// U = alpha XL W.
static mr_status apply_split(const mr_apply_problem* p, int32_t count, float alpha, void* ws,
                             const std::vector<int>& order, hipStream_t s) {
  std::vector<ApplySplitLayout> lay(count);
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    lay[i] = apply_split_layout(p[i], off);
    off = lay[i].end;
  }
  char* base = static_cast<char*>(ws);
  auto half = [&](size_t o) { return reinterpret_cast<_Float16*>(base + o); };
  uint32_t* amax_all = reinterpret_cast<uint32_t*>(base + off);
  auto amax = [&](int i, int which) { return amax_all + 4 * i + which; };
  struct Src {
    const float* ptr;
    int64_t ld, rows, cols;  // of the source (transposed copies: dst rows = source columns)
    _Float16* dst;
    int64_t ldd;
    uint32_t* amax;
    int trans;
  };
  // the float32 sources of one split pass (phase 0: XR (copied transposed),
  // G, XL; phase 1: W^T)
  auto sources = [&](int i, int phase, std::vector<Src>& out) {
    const mr_apply_problem& q = p[i];
    const ApplySplitLayout& L = lay[i];
    if (phase == 0) {
      out.push_back({q.XR, q.ldxr, q.n, q.n, half(L.xr), L.n32, amax(i, 0), 1});
      out.push_back({q.G, q.ldg, q.m, q.n, half(L.g), L.n32, amax(i, 1), 0});
      out.push_back({q.XL, q.ldxl, q.m, q.m, half(L.xl), L.m32, amax(i, 2), 0});
    } else {
      out.push_back({reinterpret_cast<float*>(base + L.wt32), q.m, q.n, q.m, half(L.wt), L.m32, amax(i, 3), 0});
    }
  };
  mr_status st = MR_OK;
  auto split_pass = [&](int phase) -> mr_status {
    std::vector<Src> srcs;
    for (const int i : order) sources(i, phase, srcs);
    for (size_t k0 = 0; k0 < srcs.size(); k0 += kMaxAbsMaxJobs) {
      AbsMaxBatch b;
      memset(&b, 0, sizeof b);
      for (size_t k = k0; k < srcs.size() && b.njobs < kMaxAbsMaxJobs; ++k) {
        const Src& x = srcs[k];
        AbsMaxJob& J = b.job[b.njobs++];
        J.src = x.ptr;
        J.amax = x.amax;
        J.lds = x.ld;
        J.rows = (int32_t)x.rows;
        J.cols = (int32_t)x.cols;
        J.block_begin = b.total_blocks;
        J.vec4 = aligned(x.ptr, 16) && x.ld % 4 == 0 && x.cols % 4 == 0 ? 1 : 0;
        b.total_blocks += (int32_t)((x.rows + kAbsMaxRows - 1) / kAbsMaxRows);
      }
      mr_status r = traced(kTrApplySplit, b.total_blocks > 0, s, [&] { return launch_absmax(b, s); },
                           "apply maxima launch");
      if (r != MR_OK) return r;
    }
    for (int trans = 0; trans < 2; ++trans) {
      std::vector<const Src*> mine;
      for (const Src& x : srcs)
        if (x.trans == trans) mine.push_back(&x);
      for (size_t k0 = 0; k0 < mine.size(); k0 += kMaxSplitPadJobs) {
        SplitPadBatch b;
        memset(&b, 0, sizeof b);
        for (size_t k = k0; k < mine.size() && b.njobs < kMaxSplitPadJobs; ++k) {
          const Src& x = *mine[k];
          SplitPadJob& J = b.job[b.njobs++];
          J.src = x.ptr;
          J.dst = x.dst;
          J.amax = x.amax;
          J.lds = x.ld;
          J.ldd = x.ldd;
          J.trans = trans;
          J.block_begin = b.total_blocks;
          if (trans) {  // dst rows = source columns, valid dst columns = source rows
            J.rows = (int32_t)x.cols;
            J.cols = (int32_t)x.rows;
            J.vec4 = 0;
            b.total_blocks += tiles(x.cols, 64) * tiles(x.ldd, 64);
          } else {
            J.rows = (int32_t)x.rows;
            J.cols = (int32_t)x.cols;
            J.vec4 = aligned(x.ptr, 16) && x.ld % 4 == 0 ? 1 : 0;
            b.total_blocks += (int32_t)((x.rows * x.ldd + 2047) / 2048);
          }
        }
        mr_status r = traced(kTrApplySplit, b.total_blocks > 0, s,
                             [&] { return trans ? launch_split_pad_t(b, s) : launch_split_pad(b, s); },
                             "apply split launch");
        if (r != MR_OK) return r;
      }
    }
    return MR_OK;
  };
  auto product = [&](int stage) -> mr_status {
    X3ApplyBatch b;
    memset(&b, 0, sizeof b);
    auto flush = [&]() -> mr_status {
      if (b.njobs == 0) return MR_OK;
      mr_status r = traced(kTrApplyX3, b.total_blocks > 0, s, [&] { return launch_x3_apply(b, s); },
                           "precondition_apply launch");
      b.njobs = 0;
      b.total_blocks = 0;
      return r;
    };
    for (const int i : order) {
      const mr_apply_problem& q = p[i];
      const ApplySplitLayout& L = lay[i];
      X3ApplyJob& J = b.job[b.njobs];
      if (stage == 0) {  // W^T = XR^T G^T : n x m, contraction n
        J.a = half(L.xr);
        J.b = half(L.g);
        J.c = reinterpret_cast<float*>(base + L.wt32);
        J.a_max = amax(i, 0);
        J.b_max = amax(i, 1);
        J.ld = L.n32;
        J.ldc = q.m;
        J.M = (int32_t)q.n;
        J.N = (int32_t)q.m;
        J.alpha = 1.f;
      } else {  // U = alpha XL W : m x n, contraction m
        J.a = half(L.xl);
        J.b = half(L.wt);
        J.c = q.U;
        J.a_max = amax(i, 2);
        J.b_max = amax(i, 3);
        J.ld = L.m32;
        J.ldc = q.ldu;
        J.M = (int32_t)q.m;
        J.N = (int32_t)q.n;
        J.alpha = alpha;
      }
      J.tiles_n = tiles(J.N, 128);
      J.nblocks = tiles(J.M, 128) * J.tiles_n;
      J.block_begin = b.total_blocks;
      b.total_blocks += round8(J.nblocks);
      ++b.njobs;
      if (b.njobs == kMaxX3ApplyJobs && (st = flush()) != MR_OK) return st;
    }
    return flush();
  };
  if ((st = traced(kTrApplySplit, true, s, [&] { return launch_fill_zero(amax_all, 4 * count, s); },
                   "apply maxima clear")) != MR_OK)
    return st;
  if ((st = split_pass(0)) != MR_OK) return st;
  if ((st = product(0)) != MR_OK) return st;
  if ((st = split_pass(1)) != MR_OK) return st;
  return product(1);
}

mr_status precondition_apply(const mr_apply_problem* p, int32_t count, float alpha, void* ws, size_t ws_bytes,
                             void* hip_stream) {
  mr_status st = validate_apply(p, count, alpha);
  if (st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const size_t need = precondition_apply_workspace(p, count);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(MR_ERR_WORKSPACE, "workspace %p of %zu bytes; need %zu bytes, 256-byte aligned", ws, ws_bytes, need);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  // largest weights first in each launch (their tiles start early, small ones fill the tail)
  std::vector<int> order(count);
  for (int i = 0; i < count; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
    return p[x].m * p[x].n * (p[x].m + p[x].n) > p[y].m * p[y].n * (p[y].m + p[y].n);
  });
  return apply_split(p, count, alpha, ws, order, s);
}

// ================================================ inv_quarter_root_batched
static mr_status validate_root_problems(const mr_root_problem* p, int32_t count, mr_dtype dt) {
  const size_t es = base_dtype(dt) == MR_F64 ? 8 : 4;
  const bool packed = is_packed(dt);
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    const mr_root_problem& q = p[i];
    if (q.d < 1 || q.d > kMaxDim)
      return fail(MR_ERR_SHAPE, "problem %d: d=%lld outside [1, %lld]", i, (long long)q.d, (long long)kMaxDim);
    if (!q.A || !q.X) return fail(MR_ERR_NULL, "problem %d: A or X is NULL", i);
    if ((!packed && q.lda < q.d) || q.ldx < q.d) return fail(MR_ERR_STRIDE, "problem %d: lda or ldx < d", i);
    if (!aligned(q.A, es) || !aligned(q.X, 4)) return fail(MR_ERR_PARAM, "problem %d: A or X misaligned", i);
    if (overlap(sym_range_of(q.A, q.d, q.lda, es, packed), range_of(q.X, q.d, q.d, q.ldx, 4)))
      return fail(MR_ERR_ALIAS, "problem %d: X overlaps A", i);
    al.in(sym_range_of(q.A, q.d, q.lda, es, packed), i, "A");
    al.out(range_of(q.X, q.d, q.d, q.ldx, 4), i, "X");
  }
  return al.check();
}

static mr_status validate_root(const mr_root_problem* p, int32_t count, mr_dtype dt, double eps, int32_t normalize,
                               int32_t method) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!valid_dtype(dt))
    return fail(MR_ERR_PARAM, "a_dtype %d is not MR_F32 or MR_F64 (optionally | MR_PACKED)", dt);
  if (!(eps > 0.0) || !std::isfinite(eps)) return fail(MR_ERR_PARAM, "eps %g must be positive and finite", eps);
  if (normalize != MR_NORM_NONE && normalize != MR_NORM_TRACE)
    return fail(MR_ERR_PARAM, "normalize %d is not MR_NORM_NONE or MR_NORM_TRACE", normalize);
  if (method != MR_AUTO && method != MR_JACOBI && method != MR_NEWTON && method != MR_NEWTON_F64 &&
      method != MR_NEWTON_F32)
    return fail(MR_ERR_PARAM, "method %d unknown", method);
  mr_status st = validate_root_problems(p, count, dt);
  if (st != MR_OK) return st;
  for (int i = 0; i < count; ++i)
    if (method == MR_JACOBI && p[i].d > kJacobiMaxD)
      return fail(MR_ERR_UNSUPPORTED, "problem %d: MR_JACOBI supports d <= %d (d = %lld)", i, kJacobiMaxD,
                  (long long)p[i].d);
  return MR_OK;
}

size_t inv_quarter_root_batched_workspace(const mr_root_problem* p, int32_t count, mr_dtype, int32_t method) {
  if (!p || count <= 0) return 0;
  for (int i = 0; i < count; ++i)
    if (p[i].d < 1 || p[i].d > kMaxDim) return 0;
  return plan_root(p, count, method).total;
}

mr_status inv_quarter_root_batched(const mr_root_problem* p, int32_t count, mr_dtype dt, double eps, int32_t normalize,
                                   int32_t method, mr_root_info* info_dev, void* ws, size_t ws_bytes,
                                   void* hip_stream) {
  mr_status st = validate_root(p, count, dt, eps, normalize, method);
  if (st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const RootPlan P = plan_root(p, count, method);
  if (!ws || ws_bytes < P.total || !aligned(ws, 256))
    return fail(MR_ERR_WORKSPACE, "workspace %p of %zu bytes; need %zu bytes, 256-byte aligned", ws, ws_bytes,
                P.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  char* base = static_cast<char*>(ws);
  RootState* state = reinterpret_cast<RootState*>(base + P.state_off);
  double* partial = reinterpret_cast<double*>(base + P.partial_off);
  double* sched = reinterpret_cast<double*>(base + P.sched_off);
  const int a_f64 = base_dtype(dt) == MR_F64;
  const int a_packed = is_packed(dt) ? 1 : 0;
  const bool all_f64 = method == MR_NEWTON_F64;
  const bool f32_mfma = method == MR_NEWTON_F32;
  // Default Newton path: X in split-fp16 storage with split-fp16 products from
  // the first step; only M and its powers take float64-accurate products while
  // the floor is low (on int8 digit planes from kI8MinD).
  const bool x_low = split_path(method);

  // ---------------- Jacobi matrices: descriptors into the workspace, then one
  // launch per size class (one workgroup per matrix)
  if (P.n_newton < count) {
    JacobiDesc* table = reinterpret_cast<JacobiDesc*>(base + P.jac_desc_off);
    JacobiDescBatch db;
    memset(&db, 0, sizeof db);
    db.dst = table;
    for (int slot = P.n_newton; slot < count; ++slot) {
      const mr_root_problem& q = p[P.slot_problem[slot]];
      JacobiDesc& D = db.desc[db.count++];
      D.A = q.A;
      D.lda = q.lda;
      D.X = q.X;
      D.ldx = q.ldx;
      const size_t woff = P.jac_w_off[slot - P.n_newton];
      D.W = woff ? reinterpret_cast<double*>(base + woff) : nullptr;
      D.d = (int32_t)q.d;
      D.slot = slot;
      D.problem = P.slot_problem[slot];
      if (db.count == kMaxJacobiDesc || slot == count - 1) {
        if ((st = traced(kTrJacobi, true, s, [&] { return launch_jacobi_desc(db, s); }, "jacobi table")) != MR_OK)
          return st;
        db.first += db.count;
        db.count = 0;
      }
    }
    for (int c = 0; c < kJacobiClasses; ++c) {
      if (P.jac_count[c] == 0) continue;
      JacobiLaunch L;
      memset(&L, 0, sizeof L);
      L.desc = table;
      L.state = state;
      L.eps = eps;
      L.first = P.jac_first[c] - P.n_newton;
      L.count = P.jac_count[c];
      L.normalize = normalize;
      L.max_sweeps = g_jacobi_max_sweeps.load();
      L.a_packed = a_packed;
      if ((st = traced(kTrJacobi, true, s, [&] { return launch_jacobi(L, kJacobiClass[c], a_f64 != 0, s); },
                       "jacobi launch")) != MR_OK)
        return st;
    }
  }

  if (P.n_newton > 0) {
    // Build per-matrix batches (stats, init, finalize) over Newton slots.
    auto run_root_batches = [&](int kind) -> mr_status {
      RootBatch b;
      memset(&b, 0, sizeof b);
      b.a_f64 = a_f64;
      b.a_packed = a_packed;
      b.normalize = normalize;
      b.eps = eps;
      b.state = state;
      b.partial = partial;
      b.partial_stride = P.partial_stride;
      b.x_low = x_low ? 1 : 0;
      b.sched = sched;
      for (const auto& c : P.classes) {
        for (int k = 0; k < c.count; ++k) {
          const int slot = c.first_slot + k;
          const mr_root_problem& q = p[P.slot_problem[slot]];
          RootJob& J = b.job[b.njobs];
          J.A = q.A;
          J.lda = q.lda;
          J.X = q.X;
          J.ldx = q.ldx;
          J.region = base + c.region_off + c.matrix_bytes * (size_t)k;
          J.d = (int32_t)q.d;
          J.slot = slot;
          J.problem = P.slot_problem[slot];
          J.block_begin = b.total_blocks;
          const bool moment = q.d >= kMomentMinD;
          if (kind == 0)
            J.nblocks = tiles(q.d, kStatsRows);
          else if (kind == 1)
            J.nblocks = upper_tiles(q.d, 32);
          else if (kind == 3)  // fp16 copy for the fourth-moment bound
            J.nblocks = moment ? upper_tiles(moment_pad((int)q.d), 32) : 0;
          else if (kind == 4 || kind == 5)  // tile sums of its square (4) and fourth power (5)
            J.nblocks = moment ? moment_tiles((int)q.d) : 0;
          else
            J.nblocks = tiles(q.d, kFinalRows);
          b.total_blocks += J.nblocks;
          ++b.njobs;
          if (b.njobs == kMaxRootJobs || slot == P.n_newton - 1) {
            const int cls = kind == 0 ? kTrStats : kind == 1 ? kTrInit : kind >= 3 ? kTrMoment : kTrFinalize;
            mr_status r = traced(cls, b.total_blocks > 0, s, [&] {
              switch (kind) {
                case 0: return launch_root_stats(b, s);
                case 1: return launch_root_init(b, s);
                case 3: return launch_root_moment_convert(b, s);
                case 4: return launch_root_moment(b, 0, s);
                case 5: return launch_root_moment(b, 1, s);
                default: return launch_root_finalize(b, s);
              }
            }, "root launch");
            if (r != MR_OK) return r;
            b.njobs = 0;
            b.total_blocks = 0;
          }
        }
      }
      return MR_OK;
    };

    if ((st = run_root_batches(0)) != MR_OK) return st;

    // Iteration cap known on the host, so the call never waits for the
    // device.  Trace mode: c <= 1.01 (1 + eps) up to rounding, so no matrix
    // needs more steps than the schedule from the floor eps / (1.02 (1 + eps)).
    // No rescale: the bound c is only known on the device; the cap is the
    // schedule from the floor kNoneFloorCap, every matrix runs its own
    // schedule under it (the launches past its last step exit at once), and
    // one whose floor eps / c lies lower runs the cap's schedule itself,
    // flagged MR_INFO_NOT_CONVERGED.  Both rely on the step count and the
    // float64 step count never rising with the floor.
    int k_cap, j_cap;
    const double floor_cap = normalize == MR_NORM_TRACE ? eps / (1.02 * (1.0 + eps)) : kNoneFloorCap;
    newton_scaled_schedule(floor_cap, 1.0 / kBoundSafety, kNewtonTol, kSwitchM, kMaxNewtonIters, nullptr, &k_cap,
                           &j_cap, x_low);
    if ((st = traced(kTrBound, true, s, [&] {
           return launch_root_bound(state, partial, P.partial_stride, sched, 0, P.n_newton, normalize, eps, k_cap,
                                    floor_cap, all_f64 ? 1 : 0, x_low ? 1 : 0, s);
         }, "root bound launch")) != MR_OK)
      return st;
    // The fourth-moment bound where it is tighter: a higher floor, fewer steps
    // (never more: the host's count above still covers every matrix).
    int64_t dmax_newton_call = 0;
    for (const auto& c : P.classes) dmax_newton_call = std::max<int64_t>(dmax_newton_call, c.d);
    if (dmax_newton_call >= kMomentMinD) {
      if ((st = run_root_batches(3)) != MR_OK) return st;
      if ((st = run_root_batches(4)) != MR_OK) return st;
      if ((st = run_root_batches(5)) != MR_OK) return st;
      if ((st = traced(kTrMoment, true, s, [&] {
             return launch_root_tighten(state, partial, P.partial_stride, sched, 0, P.n_newton, eps, k_cap, floor_cap,
                                        all_f64 ? 1 : 0, x_low ? 1 : 0, s);
           }, "root tighten launch")) != MR_OK)
        return st;
    }
    const int k_max = k_cap, j_max = all_f64 ? k_cap : j_cap;
    if ((st = run_root_batches(1)) != MR_OK) return st;

    // Class groups: at most kMaxClasses per launch, split by vector width.
    // vec64: float64 loads of 2 (d even); vec32: float32 loads of 4 (d % 4 == 0);
    // vecx3: fp16 loads of 8 (d % 8 == 0).
    // wide: d % 32 == 0 and d >= kWideMinD, the split-fp16 stages run on 256 x 256 tiles.
    // i8: the float64 steps' products on int8 digit planes (split path, d >= kI8MinD).
    struct Group {
      std::vector<int> cls;
      int vec64, vec32, vecx3;
      bool wide, i8;
    };
    std::vector<Group> groups;
    for (const int align : {32, 8, 4, 2, 1})
      for (const bool big : {true, false}) {
        Group g;
        g.vec64 = align >= 2 ? 2 : 1;
        g.vec32 = align >= 4 ? 4 : 1;
        g.vecx3 = align >= 8 ? 8 : 1;
        g.wide = align == 32;  // split-fp16 stages on 256 x 256 tiles
        g.i8 = x_low && big;
        for (int ci = 0; ci < (int)P.classes.size(); ++ci) {
          const int64_t d = P.classes[ci].d;
          const int a = d % 32 == 0 && d >= kWideMinD ? 32 : d % 8 == 0 ? 8 : d % 4 == 0 ? 4 : d % 2 == 0 ? 2 : 1;
          if (a != align || (d >= kI8MinD) != big) continue;
          g.cls.push_back(ci);
          if ((int)g.cls.size() == kMaxClasses) {
            groups.push_back(g);
            g.cls.clear();
          }
        }
        if (!g.cls.empty()) groups.push_back(g);
      }
    // tile: 256 for the wide split-fp16 kernel, else 128
    auto make_launch = [&](const Group& g, int kind, int stage, int t, int job_only, int tile = 128) {
      NewtonLaunch L;
      memset(&L, 0, sizeof L);
      L.stage = stage;
      L.t = t;
      L.state = state;
      L.sched = sched;
      L.x_low = x_low ? 1 : 0;
      L.job_only = job_only;
      L.wide = tile == 256 ? 1 : 0;
      // Largest Grams first: their long tiles start early and the short
      // tiles of the small classes fill the launch's tail.
      for (size_t q = 0; q < g.cls.size(); ++q) {
        const int ci = g.cls[g.cls.size() - 1 - q];
        const auto& c = P.classes[ci];
        NewtonClass& C = L.cls[L.ncls++];
        C.region = base + c.region_off;
        C.matrix_bytes = (int64_t)c.matrix_bytes;
        C.d = (int32_t)c.d;
        C.count = c.count;
        C.T = tiles(c.d, tile);
        C.U = C.T * (C.T + 1) / 2;
        C.slot_begin = c.first_slot;
        C.block_begin = L.total_blocks;
        if (kind == 0)
          C.blocks_per_matrix = (stage == 0 && job_only < 0 ? 2 : 1) * C.U;
        else if (kind == 2)
          C.blocks_per_matrix = (int32_t)(oz_pad(c.d) / kOzSliceRows);  // digit planes of M: a wave per padded row
        else
          C.blocks_per_matrix = (int32_t)((c.d * c.d + 2047) / 2048);
        C.nblocks = C.blocks_per_matrix * C.count;
        L.total_blocks += round8(C.nblocks);
      }
      return L;
    };
    for (int t = 0; t < k_max; ++t) {
      if (t <= j_max && !all_f64) {
        for (const auto& g : groups)
          if ((st = traced(kTrConvert, true, s, [&] { return launch_newton_convert(make_launch(g, 1, 0, t, -1), s); },
                           "newton convert")) != MR_OK)
            return st;
      }
      if (t < j_max) {  // digit planes of M
        for (const auto& g : groups)
          if (g.i8 && (st = traced(kTrSlice, true, s,
                                   [&] { return launch_newton_slice(make_launch(g, 2, 0, t, -1), s); },
                                   "newton slice")) != MR_OK)
            return st;
      }
      for (int stage = 0; stage < 3; ++stage) {
        for (const auto& g : groups) {
          if (t < j_max) {
            // float64 steps; with x_low the X update goes to the split-fp16
            // kernel, and from kI8MinD the products run on digit planes
            const bool split = x_low && stage == 0;
            const NewtonLaunch L64 = make_launch(g, 0, stage, t, split ? 0 : -1);
            if ((st = traced(g.i8 ? kTrNewtonI8 : kTrNewton64, true, s,
                             [&] { return launch_newton_stage(L64, g.i8 ? kStageI8 : kStageF64, g.vec64, s); },
                             "newton f64 stage")) != MR_OK)
              return st;
            if (split && t > 0) {  // the first X update is part of the init
              const NewtonLaunch LX = make_launch(g, 0, stage, t, 1, g.wide ? 256 : 128);
              if ((st = traced(kTrNewtonX3, true, s, [&] { return launch_newton_stage(LX, kStageX3B64, g.vecx3, s); },
                               "newton x3 X update")) != MR_OK)
                return st;
            }
          }
          if (!all_f64) {
            const NewtonLaunch L = make_launch(g, 0, stage, t, -1, g.wide && !f32_mfma ? 256 : 128);
            const int kind = f32_mfma ? kStageF32 : kStageX3;
            if ((st = traced(f32_mfma ? kTrNewton32 : kTrNewtonX3, true, s,
                             [&] { return launch_newton_stage(L, kind, f32_mfma ? g.vec32 : g.vecx3, s); },
                             "newton f32 stage")) != MR_OK)
              return st;
          }
        }
      }
    }
    if ((st = run_root_batches(2)) != MR_OK) return st;
  }

  return traced(kTrInfo, true, s, [&] { return launch_root_info(state, partial, P.partial_stride, count, info_dev, s); },
                "root info");
}

}  // extern "C"

// ================================== inv_quarter_root_batched_noalloc
// The same call with the workspace in a file-scope device array instead of a
// caller buffer, for callers that cannot allocate device memory.  In host
// code `scratch` names a host-side stand-in, so its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[MR_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;  // device ordinal -> address of its copy of `scratch`

mr_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_addr.find(dev);
  if (it != g_scratch_addr.end()) {
    *out = it->second;
    return MR_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!ptr || !aligned(ptr, 256)) return fail(MR_ERR_HIP, "scratch array at %p is not 256-byte aligned", ptr);
  g_scratch_addr.emplace(dev, ptr);
  *out = ptr;
  return MR_OK;
}
}  // namespace

extern "C" {

mr_status inv_quarter_root_batched_noalloc(const mr_root_problem* p, int32_t count, mr_dtype dt, double eps,
                                           int32_t normalize, int32_t method, mr_root_info* info_dev,
                                           void* hip_stream) {
  mr_status st = validate_root(p, count, dt, eps, normalize, method);
  if (st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const size_t need = plan_root(p, count, method).total;
  if (need > (size_t)MR_NOALLOC_SCRATCH_BYTES)
    return fail(MR_ERR_WORKSPACE,
                "inv_quarter_root_batched_noalloc: this batch needs %zu bytes of workspace, more than the %zu-byte "
                "scratch array; call inv_quarter_root_batched with a workspace instead",
                need, (size_t)MR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MR_OK) return st;
  return inv_quarter_root_batched(p, count, dt, eps, normalize, method, info_dev, ws, MR_NOALLOC_SCRATCH_BYTES,
                                  hip_stream);
}

}  // extern "C"

// ================================================ inv_sqrt_root_batched
namespace {

const CansCeilings& cans_ceilings() {
  static const CansCeilings c = cans_ceilings_compute();
  return c;
}
const CansScales& cans_scales() {
  static const CansScales s = cans_scales_from(cans_ceilings());
  return s;
}

struct CansPlan {
  std::vector<int> slot_problem;  // slots grouped by d, ascending
  std::vector<RootPlan::Cls> classes;
  size_t state_off = 0, partial_off = 0, total = 0;
  int64_t partial_stride = 0;
};

CansPlan plan_cans(const mr_root_problem* p, int32_t count) {
  CansPlan P;
  std::map<int64_t, std::vector<int>> by_d;
  for (int i = 0; i < count; ++i) by_d[p[i].d].push_back(i);
  int64_t dmax = 1;
  for (auto& kv : by_d) {
    RootPlan::Cls c;
    c.d = kv.first;
    c.first_slot = (int)P.slot_problem.size();
    c.count = (int)kv.second.size();
    c.matrix_bytes = align256((size_t)cans_matrix_bytes(c.d));
    for (int i : kv.second) P.slot_problem.push_back(i);
    P.classes.push_back(c);
    dmax = std::max(dmax, c.d);
  }
  size_t off = 0;
  P.state_off = off;
  off = align256(off + sizeof(RootState) * (size_t)std::max(count, 1));
  P.partial_stride = std::max<int64_t>(3 * ((dmax + kStatsRows - 1) / kStatsRows), (dmax + kFinalRows - 1) / kFinalRows);
  P.partial_off = off;
  off = align256(off + sizeof(double) * (size_t)P.partial_stride * (size_t)std::max(count, 1));
  for (auto& c : P.classes) {
    c.region_off = off;
    off += c.matrix_bytes * (size_t)c.count;
  }
  P.total = off;
  return P;
}

}  // namespace

extern "C" {

int32_t mr_cans_ceilings(double* y, double* z, double* p, int32_t capacity) {
  const CansCeilings& c = cans_ceilings();
  const int n = std::min(std::max(capacity, 0), kCansSteps + 1);
  for (int k = 0; k < n; ++k) {
    if (y) y[k] = c.y[k];
    if (z) z[k] = c.z[k];
    if (p) p[k] = c.p[k];
  }
  return kCansSteps + 1;
}

size_t inv_sqrt_root_batched_workspace(const mr_root_problem* p, int32_t count, mr_dtype, int32_t) {
  if (!p || count <= 0) return 0;
  for (int i = 0; i < count; ++i)
    if (p[i].d < 1 || p[i].d > kMaxDim) return 0;
  return plan_cans(p, count).total;
}

mr_status inv_sqrt_root_batched(const mr_root_problem* p, int32_t count, mr_dtype dt, double eps, int32_t normalize,
                                int32_t precision, mr_root_info* info_dev, void* ws, size_t ws_bytes,
                                void* hip_stream) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!valid_dtype(dt))
    return fail(MR_ERR_PARAM, "a_dtype %d is not MR_F32 or MR_F64 (optionally | MR_PACKED)", dt);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(MR_ERR_PARAM, "eps %g must be >= 0 and finite", eps);
  if (normalize != MR_NORM_NONE && normalize != MR_NORM_TRACE)
    return fail(MR_ERR_PARAM, "normalize %d is not MR_NORM_NONE or MR_NORM_TRACE", normalize);
  if (precision != MR_CANS_F16 && precision != MR_CANS_SPLIT)
    return fail(MR_ERR_PARAM, "precision %d is not MR_CANS_F16 or MR_CANS_SPLIT", precision);
  mr_status st = validate_root_problems(p, count, dt);
  if (st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const CansPlan P = plan_cans(p, count);
  if (!ws || ws_bytes < P.total || !aligned(ws, 256))
    return fail(MR_ERR_WORKSPACE, "workspace %p of %zu bytes; need %zu bytes, 256-byte aligned", ws, ws_bytes,
                P.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  char* base = static_cast<char*>(ws);
  RootState* state = reinterpret_cast<RootState*>(base + P.state_off);
  double* partial = reinterpret_cast<double*>(base + P.partial_off);
  const CansScales& sc = cans_scales();
  const int prec = precision == MR_CANS_SPLIT ? 3 : 1;

  // per-matrix batches: 0 statistics, 1 init, 2 finalize
  auto run_batches = [&](int kind) -> mr_status {
    RootBatch b;
    memset(&b, 0, sizeof b);
    b.a_f64 = base_dtype(dt) == MR_F64;
    b.a_packed = is_packed(dt) ? 1 : 0;
    b.normalize = normalize;
    b.eps = eps;
    b.state = state;
    b.partial = partial;
    b.partial_stride = P.partial_stride;
    for (const auto& c : P.classes) {
      for (int k = 0; k < c.count; ++k) {
        const int slot = c.first_slot + k;
        const mr_root_problem& q = p[P.slot_problem[slot]];
        RootJob& J = b.job[b.njobs];
        J.A = q.A;
        J.lda = q.lda;
        J.X = q.X;
        J.ldx = q.ldx;
        J.region = base + c.region_off + c.matrix_bytes * (size_t)k;
        J.d = (int32_t)q.d;
        J.slot = slot;
        J.problem = P.slot_problem[slot];
        J.block_begin = b.total_blocks;
        J.nblocks = kind == 0 ? tiles(q.d, kStatsRows) : kind == 1 ? upper_tiles(q.d, 32) : tiles(q.d, kFinalRows);
        b.total_blocks += J.nblocks;
        ++b.njobs;
        if (b.njobs == kMaxRootJobs || slot == count - 1) {
          const int cls = kind == 0 ? kTrStats : kind == 1 ? kTrCansInit : kTrCansFinal;
          mr_status r = traced(cls, b.total_blocks > 0, s, [&] {
            if (kind == 0) return launch_root_stats(b, s);
            if (kind == 1)
              return launch_cans_init(b, sc.sy[0], sc.sz[1] * kCansCoeff[0][0], sc.sz[1] * kCansCoeff[0][1], s);
            return launch_cans_finalize(b, 1.0 / sc.sp[kCansSteps - 1], s);
          }, "cans batch launch");
          if (r != MR_OK) return r;
          b.njobs = 0;
          b.total_blocks = 0;
        }
      }
    }
    return MR_OK;
  };

  if ((st = run_batches(0)) != MR_OK) return st;
  if ((st = traced(kTrCansBound, true, s, [&] {
         return launch_cans_bound(state, partial, P.partial_stride, count, normalize, eps, sc.sz[kCansSteps], s);
       }, "cans bound launch")) != MR_OK)
    return st;
  if ((st = run_batches(1)) != MR_OK) return st;

  // size-class groups: at most kMaxClasses per launch, split by fp16 vector width
  struct Group {
    std::vector<int> cls;
    int vec;
  };
  std::vector<Group> groups;
  for (const int vec : {8, 1}) {
    Group g;
    g.vec = vec;
    for (int ci = 0; ci < (int)P.classes.size(); ++ci) {
      if ((P.classes[ci].d % 8 == 0 ? 8 : 1) != vec) continue;
      g.cls.push_back(ci);
      if ((int)g.cls.size() == kMaxClasses) {
        groups.push_back(g);
        g.cls.clear();
      }
    }
    if (!g.cls.empty()) groups.push_back(g);
  }
  // sprec: the products' precision for this stage (3 split, 1 fp16)
  auto launch_stage = [&](int stage, int k, double a0, double b0, double a1, double b1, int sprec) -> mr_status {
    for (const auto& g : groups) {
      CansLaunch L;
      memset(&L, 0, sizeof L);
      L.state = state;
      L.stage = stage;
      L.k = k;
      L.alpha[0] = a0;
      L.beta[0] = b0;
      L.alpha[1] = a1;
      L.beta[1] = b1;
      for (int ci : g.cls) {
        const auto& c = P.classes[ci];
        CansClass& C = L.cls[L.ncls++];
        C.region = base + c.region_off;
        C.matrix_bytes = (int64_t)c.matrix_bytes;
        C.d = (int32_t)c.d;
        C.count = c.count;
        C.T = tiles(c.d, cans_tile(sprec));
        C.U = C.T * (C.T + 1) / 2;
        C.slot_begin = c.first_slot;
        C.block_begin = L.total_blocks;
        C.blocks_per_matrix = stage == kCansP ? C.T * C.T : stage == kCansYZ ? 2 * C.U : C.U;
        C.nblocks = C.blocks_per_matrix * C.count;
        L.total_blocks += round8(C.nblocks);
      }
      const int cls = stage == kCansP ? kTrCansP : kTrCansYZ;
      mr_status r = traced(cls, true, s, [&] { return launch_cans_gemm(L, g.vec, sprec, s); }, "cans gemm launch");
      if (r != MR_OK) return r;
    }
    return MR_OK;
  };
  // k = 0: P_0 = Y_0, so Z_1 = Q_0 (written by the init) and Y_1 = a0 Y0 + b0 Y0^2.
  // Always a split product: near the top of the spectrum a0 y + b0 y^2 is
  // about y / 18, so an fp16 rounding of Y0 would enter 18-fold; in split
  // form Y1 is float32-accurate and the later fp16 steps see no cancellation.
  {
    const double a = kCansCoeff[0][0], b = kCansCoeff[0][1];
    if ((st = launch_stage(kCansY1, 0, b * sc.sy[1] / (sc.sy[0] * sc.sy[0]), a * sc.sy[1] / sc.sy[0], 0.0, 0.0,
                           3)) != MR_OK)
      return st;
  }
  for (int k = 1; k < kCansSteps; ++k) {
    const double a = kCansCoeff[k][0], b = kCansCoeff[k][1];
    if ((st = launch_stage(kCansP, k, sc.sp[k] / (sc.sz[k] * sc.sy[k]), 0.0, 0.0, 0.0, prec)) != MR_OK) return st;
    const double ay = b * sc.sy[k + 1] / (sc.sy[k] * sc.sp[k]), by = a * sc.sy[k + 1] / sc.sy[k];
    const double az = b * sc.sz[k + 1] / (sc.sz[k] * sc.sp[k]), bz = a * sc.sz[k + 1] / sc.sz[k];
    if ((st = launch_stage(k + 1 < kCansSteps ? kCansYZ : kCansZ, k, ay, by, az, bz, prec)) != MR_OK) return st;
  }
  if ((st = run_batches(2)) != MR_OK) return st;
  return traced(kTrCansInfo, true, s, [&] {
    return launch_cans_info(state, partial, P.partial_stride, count, info_dev, kCansResidualRms, s);
  }, "cans info");
}

}  // extern "C"

// ================================================ polar_cans_batched
namespace {

struct PolarPlan {
  struct Cls {
    int64_t M, N;
    int first_slot, count;
    size_t region_off, matrix_bytes;
  };
  std::vector<int> slot_problem;  // slots grouped by (M, N)
  std::vector<Cls> classes;
  size_t state_off = 0, partial_off = 0, total = 0;
  int64_t partial_stride = 0;
};

PolarPlan plan_polar(const mr_polar_problem* p, int32_t count) {
  PolarPlan P;
  std::map<std::pair<int64_t, int64_t>, std::vector<int>> by_shape;
  int64_t mmax = 1;
  for (int i = 0; i < count; ++i) {
    by_shape[{std::max(p[i].m, p[i].n), std::min(p[i].m, p[i].n)}].push_back(i);
    mmax = std::max(mmax, p[i].m);
  }
  for (auto& kv : by_shape) {
    PolarPlan::Cls c;
    c.M = kv.first.first;
    c.N = kv.first.second;
    c.first_slot = (int)P.slot_problem.size();
    c.count = (int)kv.second.size();
    c.matrix_bytes = align256((size_t)polar_matrix_bytes(c.M, c.N));
    for (int i : kv.second) P.slot_problem.push_back(i);
    P.classes.push_back(c);
  }
  size_t off = 0;
  P.state_off = off;
  off = align256(off + sizeof(RootState) * (size_t)std::max(count, 1));
  P.partial_stride = 3 * ((mmax + kFinalRows - 1) / kFinalRows);
  P.partial_off = off;
  off = align256(off + sizeof(double) * (size_t)P.partial_stride * (size_t)std::max(count, 1));
  for (auto& c : P.classes) {
    c.region_off = off;
    off += c.matrix_bytes * (size_t)c.count;
  }
  P.total = off;
  return P;
}

}  // namespace

extern "C" {

static mr_status validate_polar(const mr_polar_problem* p, int32_t count, int32_t precision) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (precision != MR_CANS_F16 && precision != MR_CANS_SPLIT)
    return fail(MR_ERR_PARAM, "precision %d is not MR_CANS_F16 or MR_CANS_SPLIT", precision);
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    const mr_polar_problem& q = p[i];
    if (q.m < 1 || q.n < 1 || q.m > kMaxDim || q.n > kMaxDim)
      return fail(MR_ERR_SHAPE, "problem %d: m=%lld n=%lld outside [1, %lld]", i, (long long)q.m, (long long)q.n,
                  (long long)kMaxDim);
    if (!q.G || !q.O) return fail(MR_ERR_NULL, "problem %d: G or O is NULL", i);
    if (q.ldg < q.n || q.ldo < q.n) return fail(MR_ERR_STRIDE, "problem %d: ldg or ldo < n", i);
    if (!aligned(q.G, 4) || !aligned(q.O, 4)) return fail(MR_ERR_PARAM, "problem %d: G or O misaligned", i);
    if (overlap(range_of(q.G, q.m, q.n, q.ldg, 4), range_of(q.O, q.m, q.n, q.ldo, 4)))
      return fail(MR_ERR_ALIAS, "problem %d: O overlaps G", i);
    al.in(range_of(q.G, q.m, q.n, q.ldg, 4), i, "G");
    al.out(range_of(q.O, q.m, q.n, q.ldo, 4), i, "O");
  }
  return al.check();
}

size_t polar_cans_batched_workspace(const mr_polar_problem* p, int32_t count, int32_t) {
  if (!p || count <= 0) return 0;
  for (int i = 0; i < count; ++i)
    if (p[i].m < 1 || p[i].n < 1 || p[i].m > kMaxDim || p[i].n > kMaxDim) return 0;
  return plan_polar(p, count).total;
}

mr_status polar_cans_batched(const mr_polar_problem* p, int32_t count, int32_t precision, mr_root_info* info_dev,
                             void* ws, size_t ws_bytes, void* hip_stream) {
  mr_status st = validate_polar(p, count, precision);
  if (st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const PolarPlan P = plan_polar(p, count);
  if (!ws || ws_bytes < P.total || !aligned(ws, 256))
    return fail(MR_ERR_WORKSPACE, "workspace %p of %zu bytes; need %zu bytes, 256-byte aligned", ws, ws_bytes,
                P.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  char* base = static_cast<char*>(ws);
  RootState* state = reinterpret_cast<RootState*>(base + P.state_off);
  double* partial = reinterpret_cast<double*>(base + P.partial_off);
  const CansCeilings& ce = cans_ceilings();
  double sx[kCansSteps + 1], sa[kCansSteps + 1];
  for (int k = 0; k <= kCansSteps; ++k) {
    sx[k] = cans_pow2_scale(std::sqrt(ce.p[k]));
    sa[k] = cans_pow2_scale(ce.p[k]);
  }
  const int prec = precision == MR_CANS_SPLIT ? 3 : 1;

  // per-matrix batches: 0 statistics, 1 init, 2 finalize
  auto run_batches = [&](int kind) -> mr_status {
    PolarBatch b;
    memset(&b, 0, sizeof b);
    b.state = state;
    b.partial = partial;
    b.partial_stride = P.partial_stride;
    for (const auto& c : P.classes) {
      for (int k = 0; k < c.count; ++k) {
        const int slot = c.first_slot + k;
        const mr_polar_problem& q = p[P.slot_problem[slot]];
        PolarJob& J = b.job[b.njobs];
        J.G = q.G;
        J.ldg = q.ldg;
        J.O = q.O;
        J.ldo = q.ldo;
        J.region = base + c.region_off + c.matrix_bytes * (size_t)k;
        J.m = (int32_t)q.m;
        J.n = (int32_t)q.n;
        J.slot = slot;
        J.problem = P.slot_problem[slot];
        J.block_begin = b.total_blocks;
        J.nblocks = kind == 1 ? tiles(q.m, 32) * tiles(q.n, 32) : tiles(q.m, kFinalRows);
        b.total_blocks += J.nblocks;
        ++b.njobs;
        if (b.njobs == kMaxRootJobs || slot == count - 1) {
          const int cls = kind == 0 ? kTrPolarStats : kind == 1 ? kTrPolarInit : kTrPolarFinal;
          mr_status r = traced(cls, b.total_blocks > 0, s, [&] {
            if (kind == 0) return launch_polar_stats(b, s);
            if (kind == 1) return launch_polar_init(b, sx[0], s);
            return launch_polar_finalize(b, 1.0 / sa[kCansSteps - 1], s);
          }, "polar batch launch");
          if (r != MR_OK) return r;
          b.njobs = 0;
          b.total_blocks = 0;
        }
      }
    }
    return MR_OK;
  };

  if ((st = run_batches(0)) != MR_OK) return st;
  if ((st = traced(kTrPolarBound, true, s, [&] {
         return launch_polar_bound(state, partial, P.partial_stride, count, 1.0 / sx[kCansSteps], s);
       }, "polar bound launch")) != MR_OK)
    return st;
  if ((st = run_batches(1)) != MR_OK) return st;

  struct Group {
    std::vector<int> cls;
    int vec;
  };
  std::vector<Group> groups;
  for (const int vec : {8, 1}) {
    Group g;
    g.vec = vec;
    for (int ci = 0; ci < (int)P.classes.size(); ++ci) {
      const auto& c = P.classes[ci];
      if (((c.M % 8 == 0 && c.N % 8 == 0) ? 8 : 1) != vec) continue;
      g.cls.push_back(ci);
      if ((int)g.cls.size() == kMaxClasses) {
        groups.push_back(g);
        g.cls.clear();
      }
    }
    if (!g.cls.empty()) groups.push_back(g);
  }
  for (int k = 0; k < kCansSteps; ++k) {
    const double a = kCansCoeff[k][0], b = kCansCoeff[k][1];
    for (const int stage : {(int)kPolarA, (int)kPolarX}) {
      for (const auto& g : groups) {
        PolarLaunch L;
        memset(&L, 0, sizeof L);
        L.state = state;
        L.stage = stage;
        L.k = k;
        if (stage == kPolarA) {
          L.alpha = sa[k] / (sx[k] * sx[k]);
        } else {
          L.alpha = b * sx[k + 1] / (sx[k] * sa[k]);
          L.beta = a * sx[k + 1] / sx[k];
        }
        for (int ci : g.cls) {
          const auto& c = P.classes[ci];
          PolarClass& C = L.cls[L.ncls++];
          C.region = base + c.region_off;
          C.matrix_bytes = (int64_t)c.matrix_bytes;
          C.M = (int32_t)c.M;
          C.N = (int32_t)c.N;
          C.count = c.count;
          C.TM = tiles(c.M, polar_tile(prec, stage));
          C.TN = tiles(c.N, polar_tile(prec, stage));
          C.U = C.TN * (C.TN + 1) / 2;
          C.slot_begin = c.first_slot;
          C.block_begin = L.total_blocks;
          C.blocks_per_matrix = stage == kPolarA ? C.U : C.TM * C.TN;
          C.nblocks = C.blocks_per_matrix * C.count;
          L.total_blocks += round8(C.nblocks);
        }
        if ((st = traced(stage == kPolarA ? kTrPolarA : kTrPolarX, true, s,
                         [&] { return launch_polar_gemm(L, g.vec, prec, s); }, "polar gemm launch")) != MR_OK)
          return st;
      }
    }
  }
  if ((st = run_batches(2)) != MR_OK) return st;
  // the residual of a rank-deficient G is legitimately large: never a flag
  return traced(kTrPolarInfo, true, s, [&] {
    return launch_cans_info(state, partial, P.partial_stride, count, info_dev, HUGE_VAL, s);
  }, "polar info");
}

}  // extern "C"

// ================================================ momentum / hyperball
namespace {

// Validation shared by both streaming entry points: `out` is updated in
// place, `in` is read; m x n float32 each.
mr_status validate_stream(int i, int64_t m, int64_t n, const void* in, int64_t ld_in, const void* out, int64_t ld_out,
                          const char* in_name, const char* out_name) {
  if (m < 1 || n < 1 || m > kMaxDim || n > kMaxDim)
    return fail(MR_ERR_SHAPE, "problem %d: m=%lld n=%lld outside [1, %lld]", i, (long long)m, (long long)n,
                (long long)kMaxDim);
  if (!in || !out) return fail(MR_ERR_NULL, "problem %d: %s or %s is NULL", i, in_name, out_name);
  if (ld_in < n || ld_out < n) return fail(MR_ERR_STRIDE, "problem %d: a leading dimension < n", i);
  if (!aligned(in, 4) || !aligned(out, 4)) return fail(MR_ERR_PARAM, "problem %d: %s or %s misaligned", i, in_name, out_name);
  if (overlap(range_of(in, m, n, ld_in, 4), range_of(out, m, n, ld_out, 4)))
    return fail(MR_ERR_ALIAS, "problem %d: %s overlaps %s", i, out_name, in_name);
  return MR_OK;
}

bool stream_vec4(int64_t n, const void* in, int64_t ld_in, const void* out, int64_t ld_out) {
  return n % 4 == 0 && ld_in % 4 == 0 && ld_out % 4 == 0 && aligned(in, 16) && aligned(out, 16);
}

int64_t stream_blocks(int64_t m, int64_t n) {
  const int64_t r = stream_rows_per_block(m, n);
  return (m + r - 1) / r;
}

// Run `launch(batch, vec)` over the problems, one launch per 16 of one width.
template <class Get, class Launch>
mr_status run_stream(int32_t count, Get&& get, double* partial, int64_t stride, Launch&& launch) {
  for (const int vec : {4, 1}) {
    StreamBatch b;
    memset(&b, 0, sizeof b);
    b.partial = partial;
    b.partial_stride = stride;
    for (int i = 0; i < count; ++i) {
      StreamJob J;
      get(i, J);
      const bool v4 = stream_vec4(J.n, J.in, J.ld_in, J.inout, J.ld_inout);
      if ((vec == 4) != v4) continue;
      J.rows_per_block = stream_rows_per_block(J.m, J.n);
      J.nblocks = (int32_t)stream_blocks(J.m, J.n);
      J.block_begin = b.total_blocks;
      J.slot = i;
      J.problem = i;
      b.job[b.njobs++] = J;
      b.total_blocks += J.nblocks;
      if (b.njobs == kMaxStreamJobs) {
        mr_status r = launch(b, vec);
        if (r != MR_OK) return r;
        b.njobs = 0;
        b.total_blocks = 0;
      }
    }
    if (b.njobs > 0) {
      mr_status r = launch(b, vec);
      if (r != MR_OK) return r;
    }
  }
  return MR_OK;
}

}  // namespace

extern "C" {

mr_status momentum_ema_batched(const mr_momentum_problem* p, int32_t count, double mu, void* hip_stream) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!(mu >= 0.0 && mu < 1.0)) return fail(MR_ERR_PARAM, "mu %g not in [0, 1)", mu);
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    mr_status st = validate_stream(i, p[i].m, p[i].n, p[i].G, p[i].ldg, p[i].M, p[i].ldm, "G", "M");
    if (st != MR_OK) return st;
    al.in(range_of(p[i].G, p[i].m, p[i].n, p[i].ldg, 4), i, "G");
    al.out(range_of(p[i].M, p[i].m, p[i].n, p[i].ldm, 4), i, "M");
  }
  if (mr_status st = al.check(); st != MR_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  return run_stream(
      count,
      [&](int i, StreamJob& J) {
        memset(&J, 0, sizeof J);
        J.in = p[i].G;
        J.ld_in = p[i].ldg;
        J.inout = p[i].M;
        J.ld_inout = p[i].ldm;
        J.m = (int32_t)p[i].m;
        J.n = (int32_t)p[i].n;
      },
      nullptr, 0,
      [&](const StreamBatch& b, int vec) {
        return traced(kTrMomentum, b.total_blocks > 0, s, [&] { return launch_momentum(b, vec, mu, s); },
                      "momentum launch");
      });
}

size_t hyperball_update_batched_workspace(const mr_hyperball_problem* p, int32_t count) {
  if (!p || count <= 0) return 0;
  int64_t most = 1;
  for (int i = 0; i < count; ++i) {
    if (p[i].m < 1 || p[i].n < 1 || p[i].m > kMaxDim || p[i].n > kMaxDim) return 0;
    most = std::max(most, stream_blocks(p[i].m, p[i].n));
  }
  return align256(sizeof(double) * 3 * (size_t)most * (size_t)count);
}

mr_status hyperball_update_batched(const mr_hyperball_problem* p, int32_t count, double lr, double* norms_dev,
                                   void* ws, size_t ws_bytes, void* hip_stream) {
  if (count < 0) return fail(MR_ERR_PARAM, "count %d < 0", count);
  if (count > 0 && !p) return fail(MR_ERR_NULL, "problems is NULL");
  if (!(lr >= 0.0) || !std::isfinite(lr)) return fail(MR_ERR_PARAM, "lr %g must be >= 0 and finite", lr);
  AliasSet al;
  for (int i = 0; i < count; ++i) {
    mr_status st = validate_stream(i, p[i].m, p[i].n, p[i].U, p[i].ldu, p[i].W, p[i].ldw, "U", "W");
    if (st != MR_OK) return st;
    al.in(range_of(p[i].U, p[i].m, p[i].n, p[i].ldu, 4), i, "U");
    al.out(range_of(p[i].W, p[i].m, p[i].n, p[i].ldw, 4), i, "W");
  }
  if (mr_status st = al.check(); st != MR_OK) return st;
  if (count == 0) return MR_OK;
  const size_t need = hyperball_update_batched_workspace(p, count);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(MR_ERR_WORKSPACE, "workspace %p of %zu bytes; need %zu bytes, 256-byte aligned", ws, ws_bytes, need);
  int64_t most = 1;
  for (int i = 0; i < count; ++i) most = std::max(most, stream_blocks(p[i].m, p[i].n));
  double* partial = static_cast<double*>(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  auto get = [&](int i, StreamJob& J) {
    memset(&J, 0, sizeof J);
    J.in = p[i].U;
    J.ld_in = p[i].ldu;
    J.inout = p[i].W;
    J.ld_inout = p[i].ldw;
    J.m = (int32_t)p[i].m;
    J.n = (int32_t)p[i].n;
  };
  mr_status st = run_stream(count, get, partial, 3 * most, [&](const StreamBatch& b, int vec) {
    return traced(kTrHyperReduce, b.total_blocks > 0, s, [&] { return launch_hyperball_reduce(b, vec, s); },
                  "hyperball reduce launch");
  });
  if (st != MR_OK) return st;
  return run_stream(count, get, partial, 3 * most, [&](const StreamBatch& b, int vec) {
    return traced(kTrHyperUpdate, b.total_blocks > 0, s,
                  [&] { return launch_hyperball_update(b, vec, lr, norms_dev, s); }, "hyperball update launch");
  });
}

}  // extern "C"
