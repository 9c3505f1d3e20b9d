// Internal interface between the C ABI (bb_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_plan.hpp"

namespace bb {

hipError_t launch_pack(const void *band, int64_t ld_band, void *wband, const Geometry &g, hipStream_t st);
hipError_t launch_extract(const void *wband, const Geometry &g, void *d, void *e, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, int64_t count, uint32_t v, hipStream_t st);

// One-launch-per-step scheduler: launches nblk workgroups of nt threads for
// sweeps Rlo .. Rlo+nblk-1 of step L (cycle k = L - s R each).
// Grid-barrier scheduler: one launch of `grid` resident workgroups for the
// whole pass; steps as launch_step (`steps` of them, stagger s); sync as for
// launch_persist (status word, the claim word counts arrivals, the first
// progress line holds the barrier generation; both start at zero).
hipError_t launch_barrier(int maxm, void *wband, const Geometry &g, int b, int t, int s, int64_t nsweeps,
                          int64_t steps, uint32_t *sync, int grid, int nt, uint32_t spin_limit, hipStream_t st);
hipError_t launch_step(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                       int64_t nblk, int nt, hipStream_t st);

// Persistent scheduler for one pass: `grid` workgroups of nt threads claim the
// pass's sweeps in order; sync = the workspace's counter area (status word,
// claim counter, per-sweep progress), claim and progress zeroed beforehand.
hipError_t launch_persist(int maxm, void *wband, const Geometry &g, int b, int t, int64_t nsweeps, uint32_t *sync,
                          int grid, int nt, uint32_t wait_ticks, hipStream_t st);

// Sweep groups resident in LDS: `grid` workgroups of 64 (gmax+2) threads
// claim groups of G consecutive sweeps; each keeps a ring of W band rows in
// LDS; d is the in-group lag in half-cycles.  One launch runs a run of
// consecutive passes: the run's groups are numbered pass by pass (pass j's
// groups are base .. base+ngroups-1, its progress lines at the same indices)
// and claimed in that order, so a group only ever waits for groups claimed
// before it.  The first group of a pass loads a row once the previous pass's
// group that owns the row has released it.
constexpr int kGroupMaxWaves = 8;  // G <= 6 sweeps plus a loader and a writer wave (2 waves per SIMD: 256 VGPRs)
constexpr int kMaxRunPasses = 4;
// A pass of a run in one word (the kernel derives the rest: the lag d from
// b' = b - t, n - b' - 1 sweeps, groups of G): b | t << 13 | G << 26 |
// variant << 29; variant bit 0: register tile maxm - 1 (else maxm), bit 1:
// two rows per lane (b + t > 64).
inline uint32_t group_pass_word(int b, int t, int G, int variant) {
  return uint32_t(b) | (uint32_t(t) << 13) | (uint32_t(G) << 26) | (uint32_t(variant) << 29);
}
struct GroupRun {
  int32_t npass, total;  // passes in the run (1..kMaxRunPasses), groups over the run
  int32_t gmax, maxm;    // largest G (block = 64 (gmax+2) threads); the run's register tile family
  uint32_t pass[kMaxRunPasses];
  int32_t base[kMaxRunPasses];  // the pass's first group in the run
  // Ring rows hold a window of each working-band row (the 33-entry tile
  // family only): entries w0 .. w0 + ring_stride - 1 of the stored row; 0,
  // 0: whole rows (ring stride = the working band's stride).
  int32_t ring_stride, w0;
};
hipError_t launch_group(const GroupRun &run, void *wband, const Geometry &g, int W, uint32_t *sync, int grid,
                        uint32_t wait_ticks, hipStream_t st);

// LDS bytes one workgroup stages per cycle for a pass (b, t) with register
// tile maxm.
size_t stage_lds_bytes(int dtype, int maxm, int b, int t);
// Whether the persistent kernel stages the pass's row-half blocks in LDS.
bool persist_staged(int dtype, int maxm, int b, int t);

// Symmetric band -> tridiagonal (bb_sym.hip).  pack: user upper rows into the
// working band (fill region zeroed); persist: one pass, `grid` workgroups of
// nt threads claiming sweeps in order, sync as for launch_persist; extract:
// d = diagonal, e = first superdiagonal.
hipError_t launch_sym_pack(const void *band, int64_t ld_band, void *wband, const SymGeometry &g, hipStream_t st);
hipError_t launch_sym_persist(int maxm, void *wband, const SymGeometry &g, int b, int t, int64_t nsweeps,
                              uint32_t *sync, int grid, int nt, uint32_t wait_ticks, hipStream_t st);
hipError_t launch_sym_extract(const void *wband, const SymGeometry &g, void *d, void *e, hipStream_t st);
// The symmetric sweeps in LDS-resident groups (the k_group kernel with the
// symmetric half-cycles): run.maxm 9 or 17 (fp32 also 33) for every pass of
// the run, d = the lag in halves.
hipError_t launch_sym_group(const GroupRun &run, void *wband, const SymGeometry &g, int W, uint32_t *sync, int grid,
                            uint32_t wait_ticks, hipStream_t st);

// Singular values of the bidiagonal by bisection (bb_svals.hip).  The
// workspace holds a header {lo, hi, pivmin} in its first kSvalsHeaderBytes,
// the counts of the shared top of the bisection tree (int32, heap order, up
// to kSvalsMaxTree levels) in the next kSvalsTreeBytes, then
// svals_padded_entries(n) squared off-diagonal entries.
constexpr int kSvalsHeaderBytes = 256;
constexpr int kSvalsMaxTree = 16;
constexpr int kSvalsTreeBytes = 4 << kSvalsMaxTree;
constexpr int kPrepThreads = 1024;
constexpr int kBisectThreads = 256;
int64_t svals_padded_entries(int64_t n);
int bisect_halvings(int dtype);
hipError_t launch_gk_prep(int dtype, const void *d, const void *e, int64_t n, void *work, hipStream_t st);
// tree_levels = K shared levels counted once (0: none, <= kSvalsMaxTree);
// levels = D levels resolved per round afterwards (1..6).
hipError_t launch_svals(int dtype, int tree_levels, int levels, void *work, int64_t n, int64_t i0, int64_t i1,
                        void *sigma, hipStream_t st);

}  // namespace bb
