// C ABI of the band -> bidiagonal reduction (declared in include/bb.h):
// argument validation, planning and the host side of the schedulers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "bb.h"
#include "bb_internal.hpp"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int32_t kMaxTile = 64;  // t+1 entries per row/column held in VGPRs

bool valid_shape(int64_t n, int32_t bw, int32_t tw, int32_t dtype) {
  if (dtype != BB_F32 && dtype != BB_F64 && dtype != BB_F16) return false;
  if (n < 1 || n > kMaxN || bw < 0 || tw < 1) return false;
  if (bw > 4096) return false;
  return true;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Register tile of a pass: t+1 entries per row/column.  Tiles of exactly
// t+1 run without bounds in the inner loops for every interior cycle; other
// widths use the next larger tile with guarded loops.
int pick_maxm(int32_t t) {
  switch (t + 1) {
    case 8: case 9: case 16: case 17: case 32: case 33: case 64: case 65: return t + 1;
    default: break;
  }
  if (t + 1 <= 9) return 9;
  if (t + 1 <= 17) return 17;
  if (t + 1 <= 33) return 33;
  return 65;
}

constexpr size_t kMaxLdsBytes = 160 * 1024;  // gfx950 LDS available to one workgroup

// Every pass must fit its staged row and column blocks in LDS and its band
// in 31-bit byte offsets (buffer addressing).
bool supported(const bb::Geometry &g) {
  if (g.maxt > kMaxTile) return false;
  if (uint64_t(g.n) * uint64_t(g.stride) * uint64_t(g.esize) >= (uint64_t(1) << 31)) return false;
  for (const bb::Pass &p : bb::pass_list(g.bw, g.tw))
    if (bb::stage_lds_bytes(g.dtype, pick_maxm(p.t), p.b, p.t) > kMaxLdsBytes) return false;
  return true;
}

// Safe stagger for a pass: two cycles keep consecutive sweeps apart when the
// target bandwidth b' exceeds 1, three always do (page: three-cycle
// separation passage, R + n BW > R + 1 + BW + TW).
int32_t stagger_for(const bb::Pass &p, int32_t requested) {
  const int32_t safe = (p.b - p.t > 1) ? 2 : 3;
  return std::max(requested, safe);
}

int64_t ceil_div(int64_t a, int64_t b) {  // b > 0
  return a >= 0 ? (a + b - 1) / b : -((-a) / b);
}

bb_status hip_status(hipError_t e) { return e == hipSuccess ? BB_OK : BB_ERR_HIP; }

// Default block of the step and persistent kernels: one thread per row of
// a row half and per column of a column half (b + t + 1 each), in whole
// waves, at most 256.
int default_threads(const bb::Pass &p) { return std::min(256, std::max(64, (p.b + p.t + 1 + 63) / 64 * 64)); }
// The persistent kernel with staged row halves: its copies in and out use
// every thread, so more waves pay (measured on the n = 32768 and 65536
// workloads): 256 threads above 128 rows per block, else 128.
int staged_threads(const bb::Pass &p) { return p.b + p.t + 1 > 128 ? 256 : 128; }

bb_status run_step_pass(void *wband, const bb::Geometry &g, const bb::Pass &p, const bb_tuning &tu,
                        hipStream_t st) {
  const int maxm = pick_maxm(p.t);
  const int64_t ns = bb::sweeps_of(g.n, p);
  if (ns == 0) return BB_OK;
  const int32_t s = stagger_for(p, tu.stagger);
  int nt = tu.threads_per_block;
  if (nt == 0) nt = default_threads(p);
  const int64_t bp = p.b - p.t;
  const int64_t steps = bb::steps_of(g.n, p, s);
  for (int64_t L = 0; L < steps; ++L) {
    // sweeps with 0 <= k = L - s R < K_R: R <= L/s and
    // R (s b - 1) >= L b - (n - 2 - b')
    const int64_t rhi = std::min(ns - 1, L / s);
    const int64_t rlo = std::max<int64_t>(0, ceil_div(L * p.b - (g.n - 2 - bp), int64_t(s) * p.b - 1));
    if (rhi < rlo) continue;
    if (bb::launch_step(maxm, wband, g, p.b, p.t, L, s, rlo, rhi - rlo + 1, nt, st) != hipSuccess) return BB_ERR_HIP;
  }
  return BB_OK;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// Bound of every device-side wait: tuning.spin_limit microseconds (default
// two seconds, at most twenty), passed to the kernels in ticks of the 100 MHz
// constant clock.
constexpr int64_t kDefaultWaitUs = 2000000;
constexpr int64_t kMaxWaitUs = 20000000;
uint32_t wait_ticks(const bb_tuning &tu) {
  return uint32_t((tu.spin_limit > 0 ? tu.spin_limit : kDefaultWaitUs) * 100);
}

// The grid-barrier scheduler: one launch per pass, one resident workgroup
// per CU (at most one per sweep), the step scheduler's steps separated by a
// device-wide barrier.
bb_status run_barrier_pass(void *wband, const bb::Geometry &g, const bb::Pass &p, const bb_tuning &tu,
                           uint32_t *sync, hipStream_t st) {
  const int maxm = pick_maxm(p.t);
  const int64_t ns = bb::sweeps_of(g.n, p);
  if (ns == 0) return BB_OK;
  const int32_t s = stagger_for(p, tu.stagger);
  int nt = tu.threads_per_block;
  if (nt == 0) nt = default_threads(p);
  const int64_t grid = std::min<int64_t>(tu.max_blocks > 0 ? std::min(tu.max_blocks, device_cus()) : device_cus(), ns);
  // arrivals and the generation start at zero for every pass
  if (bb::launch_fill_u32(sync + bb::kClaim, 1, 0u, st) != hipSuccess ||
      bb::launch_fill_u32(sync + bb::kSyncHeader, bb::kLine, 0u, st) != hipSuccess)
    return BB_ERR_HIP;
  if (bb::launch_barrier(maxm, wband, g, p.b, p.t, s, ns, bb::steps_of(g.n, p, s), sync, int(grid), nt,
                         wait_ticks(tu), st) != hipSuccess)
    return BB_ERR_HIP;
  return BB_OK;
}

bb_status run_persistent_pass(void *wband, const bb::Geometry &g, const bb::Pass &p, const bb_tuning &tu,
                              uint32_t *sync, hipStream_t st) {
  const int maxm = pick_maxm(p.t);
  const int64_t ns = bb::sweeps_of(g.n, p);
  if (ns == 0) return BB_OK;
  // claim counter and per-sweep progress start at zero for every pass
  if (bb::launch_fill_u32(sync + bb::kClaim, 1, 0u, st) != hipSuccess ||
      bb::launch_fill_u32(sync + bb::kSyncHeader, ns * bb::kLine, 0u, st) != hipSuccess)
    return BB_ERR_HIP;
  int nt = tu.threads_per_block;
  if (nt == 0) nt = bb::persist_staged(g.dtype, maxm, p.b, p.t) ? staged_threads(p) : default_threads(p);
  int64_t grid = tu.max_blocks > 0 ? tu.max_blocks : 2 * int64_t(device_cus());
  grid = std::min<int64_t>(grid, ns);
  const uint32_t spin = wait_ticks(tu);
  if (bb::launch_persist(maxm, wband, g, p.b, p.t, ns, sync, int(grid), nt, spin, st) != hipSuccess)
    return BB_ERR_HIP;
  return BB_OK;
}

// Sweep groups in LDS: the largest G <= 8 whose ring fits in LDS, with the
// ring as large as LDS allows (room for the auxiliary wave to run ahead).
constexpr size_t kGroupLdsBytes = kMaxLdsBytes - 2048;  // headroom for the static control block
constexpr int kGroupMaxSweeps = bb::kGroupMaxWaves - 2;

struct GroupPlan {
  int G = 0, W = 0;          // G = 0: the pass does not fit
  int ring_stride = 0, w0 = 0;  // ring rows as windows of the band's rows (0: whole rows)
};

// Entries of a stored working-band row that pass (b, t) touches: offsets
// j - i from -t (the bulge below the diagonal) to b + t (the bulge the
// column half makes), i.e. stored entries sub - t .. sub + b + t; the window
// starts and ends on 16-byte boundaries.
void ring_window(const bb::Geometry &g, const bb::Pass &p, int *w0, int *stride) {
  const int per16 = 16 / int(g.esize);
  const int lo = int(g.sub) - p.t, hi = int(g.sub) + p.b + p.t + 1;
  *w0 = lo / per16 * per16;
  *stride = (hi - *w0 + per16 - 1) / per16 * per16;
}

// Windowed groups: passes with t = 31 (one row per lane, b + t <= 64; fp32
// and fp64) or t = 32 (two rows per lane, b + t <= 128; fp32 only: fp64's
// wider windows fit one sweep), and at least this many sweeps per group
// (fewer hand every sweep through memory, as the persistent kernel does).
constexpr int kWinMinSweeps = 2;

int64_t ring_rows_cached(int64_t n, const bb::Pass &p, int G) {
  static std::mutex mu;
  static std::map<std::tuple<int64_t, int, int, int>, int64_t> cache;
  const auto key = std::make_tuple(n, p.b, p.t, G);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const int64_t rows = bb::group_ring_rows(n, p, G);
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = rows;
  return rows;
}

GroupPlan group_plan(const bb::Geometry &g, const bb::Pass &p, int requested_g) {
  GroupPlan gp;
  const int maxm = pick_maxm(p.t);
  const bool win = maxm > 17;
  // wider tiles spill registers in the group kernel, except fp32 with one
  // row per lane on windows of the rows
  // fp32: t = 31 with one row per lane (b + t <= 64), t = 32 with two
  if (win && !((g.esize != 2 && maxm == 32 && p.b + p.t <= 64) || (g.esize == 4 && maxm == 33 && p.b + p.t <= 128)))
    return gp;
  int w0 = 0, stride = int(g.stride);
  if (win) ring_window(g, p, &w0, &stride);
  const int64_t row_bytes = int64_t(stride) * g.esize;
  const int64_t W = std::min<int64_t>(int64_t(kGroupLdsBytes) / row_bytes, g.n);
  const int lo = requested_g > 0 ? requested_g : (win ? kWinMinSweeps : 1);
  const int hi = requested_g > 0 ? requested_g : kGroupMaxSweeps;
  for (int G = hi; G >= lo; --G) {
    if (ring_rows_cached(g.n, p, G) <= W) {
      gp.G = G;
      gp.W = int(W);
      if (win) {
        gp.ring_stride = stride;
        gp.w0 = w0;
      }
      return gp;
    }
  }
  return gp;
}

// The launches of passes [first, first + count): a group launch runs a run of
// consecutive passes whose rings fit, with register tiles of one family (8/9
// or 16/17 entries); under BB_SCHED_GROUP every run is one pass.  A run also
// ends at kMaxRunPasses passes and where its groups would exceed the
// workspace's progress lines (n + 1).  Passes without sweeps are skipped.
struct LaunchItem {
  bool group = false;
  int first = 0, count = 0;  // passes [first, first + count)
  bb::GroupRun run{};
  int W = 0;
};

int tile_family(int maxm) { return maxm <= 9 ? 9 : (maxm <= 17 ? 17 : 33); }

std::vector<LaunchItem> plan_launches(const bb::Geometry &g, const std::vector<bb::Pass> &passes, int first, int count,
                                      const bb_tuning &tu) {
  std::vector<LaunchItem> out;
  const bool may_group = tu.scheduler == BB_SCHED_DEFAULT || tu.scheduler == BB_SCHED_GROUP;
#ifdef BB_PROFILE
  const bool fuse = false;  // instrumented builds run every pass in a launch of its own
#else
  const bool fuse = tu.scheduler == BB_SCHED_DEFAULT;
#endif
  const int64_t lines = g.n + 1;
  for (int i = first; i < first + count; ++i) {
    const bb::Pass &p = passes[size_t(i)];
    const int64_t ns = bb::sweeps_of(g.n, p);
    if (ns == 0) continue;
    const GroupPlan gp = may_group ? group_plan(g, p, tu.group_sweeps) : GroupPlan{};
    if (gp.G == 0) {
      LaunchItem it;
      it.first = i;
      it.count = 1;
      out.push_back(it);
      continue;
    }
    const int maxm = pick_maxm(p.t);
    const int64_t ngroups = (ns + gp.G - 1) / gp.G;
    LaunchItem *cur = out.empty() ? nullptr : &out.back();
    const bool join = fuse && cur && cur->group && cur->first + cur->count == i &&
                      cur->run.npass < bb::kMaxRunPasses && cur->run.maxm == tile_family(maxm) && cur->W == gp.W &&
                      gp.ring_stride == 0 && cur->run.ring_stride == 0 && cur->run.total + ngroups <= lines;
    if (!join) {
      out.emplace_back();
      cur = &out.back();
      cur->group = true;
      cur->first = i;
      cur->W = gp.W;
      cur->run.maxm = tile_family(maxm);
      cur->run.ring_stride = gp.ring_stride;
      cur->run.w0 = gp.w0;
    }
    const int variant = (maxm != cur->run.maxm ? 1 : 0) | (g.esize != 8 && p.b + p.t > 64 ? 2 : 0);
    cur->run.pass[cur->run.npass] = bb::group_pass_word(p.b, p.t, gp.G, variant);
    cur->run.base[cur->run.npass] = cur->run.total;
    ++cur->run.npass;
    cur->run.total += int32_t(ngroups);
    cur->run.gmax = std::max(cur->run.gmax, gp.G);
    cur->count = i - cur->first + 1;
  }
  return out;
}

bb_status run_group_launch(void *wband, const bb::Geometry &g, const LaunchItem &it, const bb_tuning &tu,
                           uint32_t *sync, hipStream_t st) {
  if (bb::launch_fill_u32(sync + bb::kClaim, 1, 0u, st) != hipSuccess ||
      bb::launch_fill_u32(sync + bb::kSyncHeader, int64_t(it.run.total) * bb::kLine, 0u, st) != hipSuccess)
    return BB_ERR_HIP;
  int64_t grid = tu.max_blocks > 0 ? tu.max_blocks : int64_t(device_cus());
  grid = std::min<int64_t>(grid, it.run.total);
  const uint32_t spin = wait_ticks(tu);
  return hip_status(bb::launch_group(it.run, wband, g, it.W, sync, int(grid), spin, st));
}

// Shared validation of the workspace-level entry points.
bb_status check_work(int64_t n, int32_t bw, int32_t tw, int32_t dtype, const void *work, size_t work_bytes,
                     bb::Geometry *g) {
  if (!valid_shape(n, bw, tw, dtype)) return BB_ERR_ARG;
  *g = bb::make_geometry(n, bw, tw, dtype);
  if (!supported(*g)) return BB_ERR_UNSUPPORTED;
  if (!work || !aligned(work, 256)) return BB_ERR_ARG;
  if (work_bytes < g->total_bytes) return BB_ERR_WORKSPACE;
  return BB_OK;
}

bb_status check_tuning(const bb_tuning *tuning, bb_tuning *tu) {
  std::memset(tu, 0, sizeof(*tu));
  if (tuning) *tu = *tuning;
  if (tu->scheduler < 0 || tu->scheduler > BB_SCHED_BARRIER) return BB_ERR_ARG;
  if (tu->stagger != 0 && (tu->stagger < 2 || tu->stagger > 64)) return BB_ERR_ARG;
  if (tu->threads_per_block != 0 && (tu->threads_per_block < 64 || tu->threads_per_block > 256 ||
                                     tu->threads_per_block % 64 != 0))
    return BB_ERR_ARG;
  if (tu->max_blocks < 0 || tu->spin_limit < 0 || tu->spin_limit > kMaxWaitUs) return BB_ERR_ARG;
  if (tu->group_sweeps < 0 || tu->group_sweeps > kGroupMaxSweeps || tu->reserved != 0) return BB_ERR_ARG;
  return BB_OK;
}

// Passes [first, first + count) in order: STEP and PERSISTENT as asked;
// GROUP and DEFAULT run the group kernel where a pass's ring fits (else
// PERSISTENT), DEFAULT with runs of such passes in one launch.
bb_status run_passes(void *work, const bb::Geometry &g, const std::vector<bb::Pass> &passes, int first, int count,
                     const bb_tuning &tu, hipStream_t st) {
  uint32_t *sync = reinterpret_cast<uint32_t *>(static_cast<char *>(work) + g.sync_offset);
  if (g.dtype == BB_F16 && (tu.scheduler == BB_SCHED_STEP || tu.scheduler == BB_SCHED_BARRIER))
    return BB_ERR_UNSUPPORTED;  // no fp16 step or barrier kernel
  bb_status rc = BB_OK;
  for (const LaunchItem &it : plan_launches(g, passes, first, count, tu)) {
    const bb::Pass &p = passes[size_t(it.first)];
    if (it.group)
      rc = run_group_launch(work, g, it, tu, sync, st);
    else if (tu.scheduler == BB_SCHED_STEP)
      rc = run_step_pass(work, g, p, tu, st);
    else if (tu.scheduler == BB_SCHED_BARRIER)
      rc = run_barrier_pass(work, g, p, tu, sync, st);
    else
      rc = run_persistent_pass(work, g, p, tu, sync, st);
    if (rc != BB_OK) return rc;
  }
  return BB_OK;
}

// Symmetric band -> tridiagonal: validation and the passes.
bool sym_supported(const bb::SymGeometry &g) {
  if (g.maxt > kMaxTile) return false;
  return uint64_t(g.n) * uint64_t(g.stride) * uint64_t(g.esize) < (uint64_t(1) << 31);
}

bb_status check_sym_work(int64_t n, int32_t bw, int32_t tw, int32_t dtype, const void *work, size_t work_bytes,
                         bb::SymGeometry *g) {
  if (!valid_shape(n, bw, tw, dtype)) return BB_ERR_ARG;
  if (dtype == BB_F16) return BB_ERR_UNSUPPORTED;
  *g = bb::make_sym_geometry(n, bw, tw, dtype);
  if (!sym_supported(*g)) return BB_ERR_UNSUPPORTED;
  if (!work || !aligned(work, 256)) return BB_ERR_ARG;
  if (work_bytes < g->total_bytes) return BB_ERR_WORKSPACE;
  return BB_OK;
}

int sym_maxm(int32_t t) {
  if (t + 1 <= 9) return 9;
  if (t + 1 <= 17) return 17;
  if (t + 1 <= 33) return 33;
  return 65;
}

int64_t sym_ring_rows_cached(int64_t n, const bb::Pass &p, int G) {
  static std::mutex mu;
  static std::map<std::tuple<int64_t, int, int, int>, int64_t> cache;
  const auto key = std::make_tuple(n, p.b, p.t, G);
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const int64_t rows = bb::sym_group_ring_rows(n, p, G);
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = rows;
  return rows;
}

// Symmetric sweep groups: register tiles 9 and 17 (fp32 also 33), the
// largest G <= 4 whose ring fits in LDS (a symmetric half-cycle does more
// work per wave than a general one; beyond four sweeps per workgroup the
// waves slow each other more than the shorter hand-offs gain: measured).
constexpr int kSymGroupDefaultSweeps = 4;

GroupPlan sym_group_plan(const bb::SymGeometry &g, const bb::Pass &p, int requested_g) {
  GroupPlan gp;
  const int maxm = sym_maxm(p.t);
  if (maxm > (g.dtype == BB_F32 ? 33 : 17)) return gp;
  const int64_t row_bytes = int64_t(g.stride) * g.esize;
  const size_t ys_bytes = size_t(kGroupMaxSweeps) * size_t(maxm) * size_t(g.esize);
  const int64_t W = std::min<int64_t>(int64_t(kGroupLdsBytes - ys_bytes) / row_bytes, g.n);
  const int lo = requested_g > 0 ? requested_g : 1;
  const int hi = requested_g > 0 ? requested_g : kSymGroupDefaultSweeps;
  for (int G = hi; G >= lo; --G) {
    if (sym_ring_rows_cached(g.n, p, G) <= W) {
      gp.G = G;
      gp.W = int(W);
      return gp;
    }
  }
  return gp;
}

bb_status run_sym_persistent_pass(void *work, const bb::SymGeometry &g, const bb::Pass &p, const bb_tuning &tu,
                                  uint32_t *sync, hipStream_t st) {
  const int64_t ns = bb::sweeps_of(g.n, p);
  if (bb::launch_fill_u32(sync + bb::kClaim, 1, 0u, st) != hipSuccess ||
      bb::launch_fill_u32(sync + bb::kSyncHeader, ns * bb::kLine, 0u, st) != hipSuccess)
    return BB_ERR_HIP;
  const int nt = tu.threads_per_block ? tu.threads_per_block : 256;
  int64_t grid = tu.max_blocks > 0 ? tu.max_blocks : 2 * int64_t(device_cus());
  grid = std::min<int64_t>(grid, ns);
  const uint32_t spin = wait_ticks(tu);
  return hip_status(bb::launch_sym_persist(sym_maxm(p.t), work, g, p.b, p.t, ns, sync, int(grid), nt, spin, st));
}

// The symmetric passes in order: the group kernel where a pass's ring fits
// (else the persistent kernel), under the default scheduler with runs of
// consecutive such passes of one register tile in one launch, as for the
// general band (plan_launches).
bb_status run_sym_passes(void *work, const bb::SymGeometry &g, const std::vector<bb::Pass> &passes,
                         const bb_tuning &tu, hipStream_t st) {
  uint32_t *sync = reinterpret_cast<uint32_t *>(static_cast<char *>(work) + g.sync_offset);
  const bool may_group = tu.scheduler == BB_SCHED_DEFAULT || tu.scheduler == BB_SCHED_GROUP;
  const bool fuse = tu.scheduler == BB_SCHED_DEFAULT;
  std::vector<LaunchItem> items;
  for (int i = 0; i < int(passes.size()); ++i) {
    const bb::Pass &p = passes[size_t(i)];
    const int64_t ns = bb::sweeps_of(g.n, p);
    if (ns == 0) continue;
    const GroupPlan gp = may_group ? sym_group_plan(g, p, tu.group_sweeps) : GroupPlan{};
    if (gp.G == 0) {
      LaunchItem it;
      it.first = i;
      it.count = 1;
      items.push_back(it);
      continue;
    }
    const int64_t ngroups = (ns + gp.G - 1) / gp.G;
    LaunchItem *cur = items.empty() ? nullptr : &items.back();
    const bool join = fuse && cur && cur->group && cur->first + cur->count == i &&
                      cur->run.npass < bb::kMaxRunPasses && cur->run.maxm == sym_maxm(p.t) && cur->W == gp.W &&
                      cur->run.total + ngroups <= g.n + 1;
    if (!join) {
      items.emplace_back();
      cur = &items.back();
      cur->group = true;
      cur->first = i;
      cur->W = gp.W;
      cur->run.maxm = sym_maxm(p.t);
    }
    cur->run.pass[cur->run.npass] = bb::group_pass_word(p.b, p.t, gp.G, 0);
    cur->run.base[cur->run.npass] = cur->run.total;
    ++cur->run.npass;
    cur->run.total += int32_t(ngroups);
    cur->run.gmax = std::max(cur->run.gmax, gp.G);
    cur->count = i - cur->first + 1;
  }
  for (const LaunchItem &it : items) {
    bb_status rc = BB_OK;
    if (it.group) {
      if (bb::launch_fill_u32(sync + bb::kClaim, 1, 0u, st) != hipSuccess ||
          bb::launch_fill_u32(sync + bb::kSyncHeader, int64_t(it.run.total) * bb::kLine, 0u, st) != hipSuccess)
        return BB_ERR_HIP;
      int64_t grid = tu.max_blocks > 0 ? tu.max_blocks : int64_t(device_cus());
      grid = std::min<int64_t>(grid, it.run.total);
      const uint32_t spin = wait_ticks(tu);
      rc = hip_status(bb::launch_sym_group(it.run, work, g, it.W, sync, int(grid), spin, st));
    } else {
      rc = run_sym_persistent_pass(work, g, passes[size_t(it.first)], tu, sync, st);
    }
    if (rc != BB_OK) return rc;
  }
  return BB_OK;
}

// Bisection of the Golub-Kahan tridiagonal: sizes, and how it is split.
constexpr int64_t kMaxSvalsN = int64_t(1) << 29;  // 2n pivots indexed in 32 bits

size_t svals_bytes(int64_t n, int32_t dtype) {
  const size_t es = dtype == BB_F64 ? 8 : 4;
  return size_t(bb::kSvalsHeaderBytes) + size_t(bb::kSvalsTreeBytes) + size_t(bb::svals_padded_entries(n)) * es;
}

// Every count is a chain of 2n dependent pivots, and one wave per SIMD keeps
// the SIMD busy, so time ~ sum over launches of rounds * max(1, waves/SIMDs).
// K shared tree levels cost one round of 2^K - 1 lanes; then D levels per
// round cost a round each, with 2^D lanes per value (one for D = 1).  The
// cheapest (K, D) wins; ties go to less work (smaller K, then smaller D).
struct SvalsSplit {
  int32_t tree, levels;
};

double split_cost(int F, double simds, int64_t values, int K, int D) {
  double cost = 0;
  if (K > 0) cost += std::max(1.0, double(((int64_t(1) << K) - 1 + 63) / 64) / simds);
  if (F > K) {
    const int64_t lanes = values * (D == 1 ? 1 : (int64_t(1) << D));
    cost += double((F - K + D - 1) / D) * std::max(1.0, double((lanes + 63) / 64) / simds);
  }
  return cost;
}

SvalsSplit pick_split(int32_t dtype, int64_t values, int32_t tree, int32_t levels) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const double simds = 4.0 * cus;
  const int F = bb::bisect_halvings(dtype == BB_F64 ? 1 : 0);
  SvalsSplit best{0, 1};
  double best_cost = -1;
  for (int32_t K = 0; K <= bb::kSvalsMaxTree; ++K) {
    if ((tree > 0 && K != tree) || (tree < 0 && K != 0)) continue;
    for (int32_t D = 1; D <= 6; ++D) {
      if (levels > 0 && D != levels) continue;
      const double c = split_cost(F, simds, values, K, D);
      if (best_cost < 0 || c < best_cost - 1e-9) {
        best = {K, D};
        best_cost = c;
      }
    }
  }
  return best;
}

}  // namespace

extern "C" {

bb_status bb_sym_workspace_bytes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, size_t *bytes) {
  if (!bytes || !valid_shape(n, bw, tw, dtype)) return BB_ERR_ARG;
  if (dtype == BB_F16) return BB_ERR_UNSUPPORTED;
  const bb::SymGeometry g = bb::make_sym_geometry(n, bw, tw, dtype);
  if (!sym_supported(g)) return BB_ERR_UNSUPPORTED;
  *bytes = g.total_bytes;
  return BB_OK;
}

bb_status bb_sym_reduce(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *d,
                        void *e, void *work, size_t work_bytes, const bb_tuning *tuning, void *stream) {
  bb::SymGeometry g;
  bb_status rc = check_sym_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK && rc != BB_ERR_WORKSPACE) return rc;
  if (!band || !d || (n > 1 && !e) || ld_band < int64_t(bw) + 1) return BB_ERR_ARG;
  if (!aligned(band, g.esize) || !aligned(d, g.esize) || (n > 1 && !aligned(e, g.esize))) return BB_ERR_ARG;
  if (rc != BB_OK) return rc;
  bb_tuning tu;
  if ((rc = check_tuning(tuning, &tu)) != BB_OK) return rc;
  if (tu.scheduler == BB_SCHED_STEP || tu.scheduler == BB_SCHED_BARRIER) return BB_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t *sync = reinterpret_cast<uint32_t *>(static_cast<char *>(work) + g.sync_offset);
  if (bb::launch_sym_pack(band, ld_band, work, g, st) != hipSuccess ||
      bb::launch_fill_u32(sync, int64_t(g.sync_words), 0u, st) != hipSuccess)
    return BB_ERR_HIP;
  if ((rc = run_sym_passes(work, g, bb::pass_list(bw, tw), tu, st)) != BB_OK) return rc;
  return hip_status(bb::launch_sym_extract(work, g, d, n > 1 ? e : nullptr, st));
}

bb_status bb_sym_export_band(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *dst,
                             void *stream) {
  if (!valid_shape(n, bw, tw, dtype) || !work || !dst) return BB_ERR_ARG;
  if (dtype == BB_F16) return BB_ERR_UNSUPPORTED;
  const bb::SymGeometry g = bb::make_sym_geometry(n, bw, tw, dtype);
  const size_t row = size_t(g.ld) * size_t(g.esize);
  return hip_status(hipMemcpy2DAsync(dst, row, work, size_t(g.stride) * size_t(g.esize), row, size_t(n),
                                     hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
}

bb_status bb_sym_device_status(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *stream) {
  if (!valid_shape(n, bw, tw, dtype) || !work) return BB_ERR_ARG;
  if (dtype == BB_F16) return BB_ERR_UNSUPPORTED;
  const bb::SymGeometry g = bb::make_sym_geometry(n, bw, tw, dtype);
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return BB_ERR_HIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, static_cast<const char *>(work) + g.sync_offset, sizeof(word), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return BB_ERR_HIP;
  return word == 0 ? BB_OK : BB_ERR_TIMEOUT;
}

bb_status bb_svals_workspace_bytes(int64_t n, int32_t dtype, size_t *bytes) {
  if (!bytes || (dtype != BB_F32 && dtype != BB_F64) || n < 0 || n > kMaxSvalsN) return BB_ERR_ARG;
  *bytes = svals_bytes(n, dtype);
  return BB_OK;
}

bb_status bb_svals(const void *d, const void *e, int64_t n, int32_t dtype, int64_t i0, int64_t i1,
                   int32_t tree_levels, int32_t levels, void *sigma, void *work, size_t work_bytes, void *stream) {
  if ((dtype != BB_F32 && dtype != BB_F64) || n < 0 || n > kMaxSvalsN) return BB_ERR_ARG;
  if (i0 < 0 || i1 < i0 || i1 > n || levels < 0 || levels > 6) return BB_ERR_ARG;
  if (tree_levels < -1 || tree_levels > bb::kSvalsMaxTree) return BB_ERR_ARG;
  if (n == 0 || i1 == i0) return BB_OK;
  const size_t es = dtype == BB_F64 ? 8 : 4;
  if (!d || (n > 1 && !e) || !sigma || !work) return BB_ERR_ARG;
  if (!aligned(d, es) || (n > 1 && !aligned(e, es)) || !aligned(sigma, es) || !aligned(work, 256))
    return BB_ERR_ARG;
  if (work_bytes < svals_bytes(n, dtype)) return BB_ERR_WORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int code = dtype == BB_F64 ? 1 : 0;
  const SvalsSplit sp = pick_split(dtype, i1 - i0, tree_levels, levels);
  if (bb::launch_gk_prep(code, d, n > 1 ? e : nullptr, n, work, st) != hipSuccess) return BB_ERR_HIP;
  return hip_status(bb::launch_svals(code, sp.tree, sp.levels, work, n, i0, i1, sigma, st));
}

bb_status bb_svals_split(int64_t values, int32_t dtype, int32_t *tree_levels, int32_t *levels) {
  if (!tree_levels || !levels || (dtype != BB_F32 && dtype != BB_F64) || values < 0) return BB_ERR_ARG;
  const SvalsSplit sp = pick_split(dtype, values, 0, 0);
  *tree_levels = sp.tree;
  *levels = sp.levels;
  return BB_OK;
}

bb_status bb_plan(int64_t n, int32_t bw, int32_t tw, int32_t dtype, bb_plan_info *out) {
  if (!out || !valid_shape(n, bw, tw, dtype)) return BB_ERR_ARG;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  bb_plan_info info;
  std::memset(&info, 0, sizeof(info));
  info.ld = g.ld;
  info.sub = g.sub;
  double bytes = 0, flops = 0;
  for (const bb::Pass &p : bb::pass_list(bw, tw)) {
    ++info.passes;
    const int64_t ns = bb::sweeps_of(n, p);
    info.sweeps += ns;
    info.steps += bb::steps_of(n, p, 3);
    for (int64_t R = 0; R < ns; ++R) {
      const int64_t K = bb::cycles_of(n, p, R);
      info.cycles += K;
      for (int64_t k = 0; k < K; ++k) {
        const bb::CycleShape cs = bb::cycle_shape(n, p, R, k);
        bytes += 2.0 * double(cs.m) * double(cs.rows + cs.cols - cs.m) * g.esize;
        // norm 2(m-1); per applied row/column: dot 2(m-1) + 2, update 2(m-1) + 1
        flops += 2.0 * (2 * (cs.m - 1)) + double(cs.rows - 1 + cs.cols - 1) * (4.0 * (cs.m - 1) + 3.0);
      }
    }
  }
  info.alg_bytes = bytes;
  info.flops = flops;
  *out = info;
  return BB_OK;
}

bb_status bb_workspace_bytes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, size_t *bytes) {
  if (!bytes || !valid_shape(n, bw, tw, dtype)) return BB_ERR_ARG;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  if (!supported(g)) return BB_ERR_UNSUPPORTED;
  *bytes = g.total_bytes;
  return BB_OK;
}

bb_status bb_pack(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *work,
                  size_t work_bytes, void *stream) {
  bb::Geometry g;
  const bb_status rc = check_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK) return rc;
  if (!band || ld_band < int64_t(bw) + 1 || !aligned(band, g.esize)) return BB_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t *sync = reinterpret_cast<uint32_t *>(static_cast<char *>(work) + g.sync_offset);
  if (bb::launch_fill_u32(sync, int64_t(g.sync_words), 0u, st) != hipSuccess) return BB_ERR_HIP;
  return hip_status(bb::launch_pack(band, ld_band, work, g, st));
}

bb_status bb_run_pass(int64_t n, int32_t bw, int32_t tw, int32_t dtype, int32_t pass, void *work, size_t work_bytes,
                      const bb_tuning *tuning, void *stream) {
  bb::Geometry g;
  bb_status rc = check_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK) return rc;
  bb_tuning tu;
  if ((rc = check_tuning(tuning, &tu)) != BB_OK) return rc;
  const std::vector<bb::Pass> passes = bb::pass_list(bw, tw);
  if (pass < 0 || pass >= int32_t(passes.size())) return BB_ERR_ARG;
  return run_passes(work, g, passes, pass, 1, tu, static_cast<hipStream_t>(stream));
}

bb_status bb_run_passes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, int32_t first, int32_t count, void *work,
                        size_t work_bytes, const bb_tuning *tuning, void *stream) {
  bb::Geometry g;
  bb_status rc = check_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK) return rc;
  bb_tuning tu;
  if ((rc = check_tuning(tuning, &tu)) != BB_OK) return rc;
  const std::vector<bb::Pass> passes = bb::pass_list(bw, tw);
  if (first < 0 || count < 0 || int64_t(first) + count > int64_t(passes.size())) return BB_ERR_ARG;
  return run_passes(work, g, passes, first, count, tu, static_cast<hipStream_t>(stream));
}

bb_status bb_launch_plan(int64_t n, int32_t bw, int32_t tw, int32_t dtype, const bb_tuning *tuning,
                         int32_t *launch_of_pass, int32_t capacity, int32_t *launches) {
  if (!valid_shape(n, bw, tw, dtype) || !launches || capacity < 0 || (capacity > 0 && !launch_of_pass))
    return BB_ERR_ARG;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  if (!supported(g)) return BB_ERR_UNSUPPORTED;
  bb_tuning tu;
  bb_status rc = check_tuning(tuning, &tu);
  if (rc != BB_OK) return rc;
  if (dtype == BB_F16 && (tu.scheduler == BB_SCHED_STEP || tu.scheduler == BB_SCHED_BARRIER))
    return BB_ERR_UNSUPPORTED;  // as bb_run_passes
  const std::vector<bb::Pass> passes = bb::pass_list(bw, tw);
  if (capacity > 0 && capacity < int32_t(passes.size())) return BB_ERR_ARG;
  const std::vector<LaunchItem> items = plan_launches(g, passes, 0, int(passes.size()), tu);
  if (capacity > 0) {
    for (size_t i = 0; i < passes.size(); ++i) launch_of_pass[i] = -1;  // no sweeps: nothing to launch
    for (size_t k = 0; k < items.size(); ++k)
      for (int i = items[k].first; i < items[k].first + items[k].count; ++i) launch_of_pass[i] = int32_t(k);
  }
  *launches = int32_t(items.size());
  return BB_OK;
}

bb_status bb_extract(const void *work, size_t work_bytes, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *d,
                     void *e, void *stream) {
  bb::Geometry g;
  const bb_status rc = check_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK) return rc;
  if (!d || (n > 1 && !e) || !aligned(d, g.esize) || (e && !aligned(e, g.esize))) return BB_ERR_ARG;
  return hip_status(bb::launch_extract(work, g, d, n > 1 ? e : nullptr, static_cast<hipStream_t>(stream)));
}

bb_status bb_reduce(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *d,
                    void *e, void *work, size_t work_bytes, const bb_tuning *tuning, void *stream) {
  // validate everything before enqueuing anything
  bb::Geometry g;
  bb_status rc = check_work(n, bw, tw, dtype, work, work_bytes, &g);
  if (rc != BB_OK && rc != BB_ERR_WORKSPACE) return rc;
  if (!band || !d || (n > 1 && !e) || ld_band < int64_t(bw) + 1) return BB_ERR_ARG;
  if (!aligned(band, g.esize) || !aligned(d, g.esize) || (e && !aligned(e, g.esize))) return BB_ERR_ARG;
  if (rc != BB_OK) return rc;
  bb_tuning tu;
  if ((rc = check_tuning(tuning, &tu)) != BB_OK) return rc;
  if ((rc = bb_pack(band, ld_band, n, bw, tw, dtype, work, work_bytes, stream)) != BB_OK) return rc;
  const std::vector<bb::Pass> passes = bb::pass_list(bw, tw);
  if ((rc = run_passes(work, g, passes, 0, int(passes.size()), tu, static_cast<hipStream_t>(stream))) != BB_OK)
    return rc;
  return bb_extract(work, work_bytes, n, bw, tw, dtype, d, e, stream);
}

}  // extern "C"

// The workspace of bb_reduce_noalloc: one array per GPU, in the library's
// code object, held until the process ends.  Host code never uses its name
// as an address (that is a host-side stand-in): each device's address comes
// from hipGetSymbolAddress, called once per device with that device current.
static __device__ __align__(256) unsigned char scratch[BB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`.
bb_status scratch_of_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BB_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BB_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BB_OK;
}

}  // namespace

extern "C" {

bb_status bb_reduce_noalloc(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype,
                            void *d, void *e, void *status, const bb_tuning *tuning, void *stream) {
  size_t need = 0;
  bb_status rc = bb_workspace_bytes(n, bw, tw, dtype, &need);
  if (rc != BB_OK) return rc;
  if (need > size_t(BB_NOALLOC_SCRATCH_BYTES)) return BB_ERR_WORKSPACE;
  void *work = nullptr;
  if ((rc = scratch_of_current_device(&work)) != BB_OK) return rc;
  if ((rc = bb_reduce(band, ld_band, n, bw, tw, dtype, d, e, work, size_t(BB_NOALLOC_SCRATCH_BYTES), tuning,
                      stream)) != BB_OK)
    return rc;
  if (!status) return BB_OK;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  return hip_status(hipMemcpyAsync(status, static_cast<const char *>(work) + g.sync_offset, sizeof(uint32_t),
                                   hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
}

bb_status bb_export_band(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *dst,
                         void *stream) {
  if (!valid_shape(n, bw, tw, dtype) || !work || !dst) return BB_ERR_ARG;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  const size_t row = size_t(g.ld) * size_t(g.esize);
  return hip_status(hipMemcpy2DAsync(dst, row, work, size_t(g.stride) * size_t(g.esize), row, size_t(n),
                                     hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
}

bb_status bb_device_status(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *stream) {
  if (!valid_shape(n, bw, tw, dtype) || !work) return BB_ERR_ARG;
  const bb::Geometry g = bb::make_geometry(n, bw, tw, dtype);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return BB_ERR_HIP;
  uint32_t word = 0;
  if (hipMemcpy(&word, static_cast<const char *>(work) + g.sync_offset, sizeof(word), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return BB_ERR_HIP;
  return word == 0 ? BB_OK : BB_ERR_TIMEOUT;
}

const char *bb_status_str(int32_t status) {
  switch (status) {
    case BB_OK: return "ok";
    case BB_ERR_ARG: return "invalid argument";
    case BB_ERR_WORKSPACE: return "workspace too small";
    case BB_ERR_HIP: return "HIP call or kernel launch failed";
    case BB_ERR_UNSUPPORTED: return "unsupported shape (tile width above 64, or band too wide for LDS staging)";
    case BB_ERR_TIMEOUT: return "device-side wait expired";
    default: return "unknown status";
  }
}

}  // extern "C"
