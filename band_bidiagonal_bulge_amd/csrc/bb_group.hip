// Sweep groups resident in LDS (gfx950): one workgroup runs G consecutive
// sweeps of a pass, one wave per sweep, on a ring of band rows held in LDS,
// plus two auxiliary waves that move rows between the ring and memory: a
// loader and a writer (separate waves, so that waiting for loads never holds
// up a write-back or a publish: vmcnt is per wave).
//
// Why: a sweep must stay a few half-cycles behind its predecessor (page
// "Accelerating Bidiagonalization of Banded Matrices through Memory-Aware
// Bulge-Chasing on GPUs", three-cycle-separation passage; page "A two-stage
// reduction on an Apple M5 Pro", section 6).  Across workgroups every such
// hand-off costs a round trip through memory; inside a workgroup it is an LDS
// counter, and the data never leaves LDS.  Only the first sweep of a group
// depends on another workgroup, and it does so by whole rows.
//
// Protocol (rows are the unit between groups):
//   * group g (sweeps R0 .. R0+G-1) publishes X_g: every row below X_g has
//     been written back by g and will not be touched by g again, and
//     X_g <= X_{g-1}.  Group g loads row i only once X_{g-1} > i, so each row
//     it reads holds the final values of all earlier sweeps, and no earlier
//     sweep touches the row afterwards (every sweep touches rows in
//     nondecreasing order).
//   * inside the group, sweep j starts half-cycle q once sweep j-1 has done
//     min(q + d, all of its) half-cycles, and publishes its final count only
//     after sweep j-1 has published its own (the rule of the persistent
//     scheduler; d = 2, 3, 4 for b' >= 3, 2, 1); for b' <= 2 a sweep needs
//     only the first part of the predecessor's half q+d-1 (see group_sweep
//     and sym_group_sweep).  Sweep 0 has no in-group predecessor: its inputs
//     are whole rows, complete when loaded.
//   * each compute wave publishes the lowest row it will still touch; rows
//     below the minimum over the group are dead: the writer writes them back
//     and publishes X_g = rows written (never above X_{g-1}: only loaded rows
//     are written, and only released rows are loaded); the loader then reuses
//     their ring slots.
// Every wait is a bounded poll; on expiry the status word is set and the
// workgroup drains (the abort flag stops every wave of the group).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_device.hpp"
#include "bb_internal.hpp"

namespace bb {
namespace {

constexpr int kGroupMaxSweeps = kGroupMaxWaves - 2;

constexpr int32_t kLoadBatchRows = 64;   // rows per loader batch: early rows are signalled early
constexpr int32_t kDrainBatchRows = 32;  // rows per writer batch of the symmetric sweeps

// Rows per writer batch of pass (b, t), each batch published on its own.
// When the last sweep of a group moves its floor up by b rows, the next
// group's first sweep waits for the lowest t + 2 of them (b' >= 2; for
// b' = 1, for the lowest one), so the first batch should hold about those
// and no more: t + 2 rounded up to 16 rows, and 16 rows for b' = 1 (fewer
// rows per batch publish sooner but add batches; these sizes were the
// fastest measured).
__device__ __forceinline__ int32_t drain_batch(int b, int t) { return b - t >= 2 ? (t + 2 + 15) / 16 * 16 : 16; }

struct GroupCtl {
  int32_t g;                         // group being run (numbered over the launch's run of passes)
  uint32_t pass_word, prev_word;     // its pass and the pass before it (group_pass_word)
  int32_t base, prev_base;           // their first groups (prev_base -1: the run's first pass)
  int32_t loaded_hi;                 // rows [R0, loaded_hi) resident in the ring
  int32_t written;                   // rows [R0, written) written back; their slots are free
  int32_t abort_;                    // a wait expired: drain
  // per sweep j, published together by one 8-byte release store:
  //   word 0: progress in steps, two per half-cycle completed plus one for a
  //   first part done ahead; word 1: lowest row the sweep will still touch
  uint64_t sweep[kGroupMaxSweeps];
};

__device__ __forceinline__ int32_t lds_load(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint64_t sweep_word(int32_t prog, int32_t floor_row) {
  return uint64_t(uint32_t(prog)) | (uint64_t(uint32_t(floor_row)) << 32);
}
__device__ __forceinline__ int32_t sweep_prog(uint64_t w) { return int32_t(uint32_t(w)); }
__device__ __forceinline__ int32_t sweep_floor(uint64_t w) { return int32_t(uint32_t(w >> 32)); }
__device__ __forceinline__ uint64_t lds_load64(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One poll of a sweep's LDS wait: false once the group has aborted (checked
// every 64 polls).  The sweeps' waits need no clock of their own: whenever
// the group makes no progress, its writer idles, and the writer's idle wait
// is bounded (aux_idle); the loader raises the abort flag when any other
// wait of the launch has expired.
__device__ __forceinline__ bool keep_waiting(uint32_t &polls, GroupCtl &ctl) {
  __builtin_amdgcn_s_sleep(1);
  return (++polls & 63u) != 0 || !lds_load(&ctl.abort_);
}

// LDS poll until the progress of a sweep reaches `need` (whole wave);
// `known` caches the last value seen, so a satisfied wait costs no LDS
// access.  False on abort.
__device__ __forceinline__ bool prog_wait(const uint64_t *w, int32_t &known, int32_t need, GroupCtl &ctl,
                                          uint32_t limit, uint32_t *status);

// LDS poll until *p >= need (whole wave).  False on abort.
__device__ __forceinline__ bool lds_wait(const int32_t *p, int32_t need, GroupCtl &ctl, uint32_t limit,
                                         uint32_t *status) {
  uint32_t polls = 0;
  while (lds_load(p) < need)
    if (!keep_waiting(polls, ctl)) return false;
  return true;
}

// Instrumented builds (-DBB_PROFILE) accumulate wall-clock ticks (100 MHz)
// per phase in registers and add them, once per sweep, with atomics to the
// 64-bit counters of the workspace's profiling line (a line of its own that
// nothing polls).  Such builds run every pass in a launch of its own.
#ifdef BB_PROFILE
struct Prof {
  uint64_t v[16] = {};
  uint64_t mark = 0;
  __device__ __forceinline__ void start() { mark = wall_clock64(); }
  __device__ __forceinline__ void tick(int slot) {
    const uint64_t now = wall_clock64();
    v[slot] += now - mark;
    mark = now;
  }
  __device__ __forceinline__ void add(int slot, uint64_t x) { v[slot] += x; }
  __device__ void flush(uint32_t *sync, int lane) {
    unsigned long long *p = reinterpret_cast<unsigned long long *>(sync + kProf);
    if (lane == 0)
      for (int i = 0; i < 16; ++i)
        if (v[i]) atomicAdd(p + i, (unsigned long long)v[i]);
  }
};
#define BB_P(stmt) stmt
#else
#define BB_P(stmt)
#endif

__device__ __forceinline__ bool prog_wait(const uint64_t *w, int32_t &known, int32_t need, GroupCtl &ctl,
                                          uint32_t limit, uint32_t *status) {
  if (known >= need) return true;
  uint32_t polls = 0;
  for (;;) {
    known = sweep_prog(lds_load64(w));
    if (known >= need) return true;
    if (!keep_waiting(polls, ctl)) return false;
  }
}

// The same for the loaded-rows bound of the ring.
__device__ __forceinline__ bool rows_wait(const int32_t *p, int32_t &known, int32_t need, GroupCtl &ctl,
                                          uint32_t spin_limit, uint32_t *status) {
  if (known >= need) return true;
  if (!lds_wait(p, need, ctl, spin_limit, status)) return false;
  known = lds_load(p);
  return true;
}

// Ring of W band rows in LDS, S elements each (the working band's row
// stride): row i lives in slot i mod W, element (i, j) at
// L[slot * S + (j - i + sub)].
template <typename T>
struct Ring {
  T *L;
  int32_t S, W, sub;
  __device__ __forceinline__ int32_t slot(int32_t i) const { return i % W; }
  __device__ __forceinline__ int32_t next(int32_t s, int32_t di) const {  // slot of row i + di, di < W
    s += di;
    return s >= W ? s - W : s;
  }
  __device__ __forceinline__ T *at(int32_t s, int32_t i, int32_t j) const { return L + s * S + (j - i + sub); }
};

// The reflector of a half from the tail sum of squares sn = sum_{j>=1} x_j^2
// (already accumulated in the contract's order) and alpha = x_0; nz false:
// identity (zero tail).  Every lane holds the same x (broadcast loads), so nz
// is taken from the first lane and every branch on it is a scalar one.
template <typename T>
__device__ __forceinline__ Refl<T> house_from(T alpha, T sn) {
  Refl<T> h;
  h.nz = __builtin_amdgcn_readfirstlane(int(sn != T(0))) != 0;
  h.beta = alpha;
  h.tau = T(0);
  h.inv = T(0);
  if (h.nz) {
    const T nrm = sqrt_(fma_(alpha, alpha, sn));
    h.beta = (alpha >= T(0)) ? -nrm : nrm;
    h.tau = div_(h.beta - alpha, h.beta);
    h.inv = div_(T(1), alpha - h.beta);
  }
  return h;
}

// Each half-cycle runs in two parts.  The first forms the reflector from the
// entries that define it (row r at columns c..ch for a row half, column c at
// rows c..ch for a column half; x[0] = alpha) and writes the pivot's final
// values (beta, then zeros).  The second applies the reflector to the other
// rows or columns.  For every half but a sweep's first, the defining entries
// were last written by the sweep's own previous half, and no other sweep
// touches them or the pivot until this half is done (the in-group lag keeps
// the predecessor d halves ahead and the successor d halves behind), so the
// first part runs right after the previous half is published, while the
// sweep waits for its predecessor; only the second part is on the chain
// between sweeps.
template <typename T, int MAXM>
struct HalfRefl {
  Refl<T> h;
  T x[MAXM];  // defining entries (x[0] unused after the reflector is formed)
};

// Row half, first part.  sr: ring slot of row r; colr = c - r + sub (column
// c within row r); FULL: m == MAXM.
template <typename T, int MAXM, bool FULL, int SC>
__device__ __forceinline__ void ring_row_prep(const Ring<T> &A, int32_t sr, int32_t colr, int32_t m, int lane,
                                              HalfRefl<T, MAXM> &P) {
  const int32_t S = SC ? SC : A.S;
  T *px = A.L + __umul24(sr, S) + colr;
#pragma unroll
  for (int j = 0; j < MAXM; ++j) P.x[j] = (FULL || j < m) ? px[j] : T(0);
  T sn = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (FULL || j < m) sn = fma_(P.x[j], P.x[j], sn);
  P.h = house_from(P.x[0], sn);
  if (lane < m) px[lane] = lane > 0 ? T(0) : P.h.beta;  // row r becomes (beta, 0, ..., 0); beta = alpha for a zero tail
}

// Wide fp64 tiles form the reflector's tail x_j * inv where it is used
// instead of holding all of it in registers (the same products).
template <typename T, int MAXM>
constexpr bool kLazyTail = sizeof(T) == 8 && MAXM >= 32;

// Row half, second part: the reflector applied from the right to rows
// r+1..ch, one lane per row (rows r+1+lane and, TWO, r+65+lane; wider bands
// loop), each row's dot product with x serial in j.  nr = ch - r.
template <typename T, int MAXM, bool FULL, bool TWO, int SC>
__device__ __forceinline__ void ring_row_apply(const Ring<T> &A, int32_t sr, int32_t colr, int32_t m, int32_t nr,
                                               int lane, const HalfRefl<T, MAXM> &P) {
  if (!P.h.nz) return;
  const int32_t S = SC ? SC : A.S;
  T *L = A.L;
  const int32_t a0 = lane + 1, a1 = lane + 65;
  const bool h0 = a0 <= nr, h1 = a1 <= nr;
  const int32_t i0 = h0 ? a0 : nr, i1 = h1 ? a1 : nr;  // inactive lanes read row ch, store nothing
  int32_t s0 = sr + i0, s1 = sr + i1;
  s0 = s0 >= A.W ? s0 - A.W : s0;
  s1 = s1 >= A.W ? s1 - A.W : s1;
  T *p0 = L + __umul24(s0, S) + (colr - i0);
  T *p1 = L + __umul24(s1, S) + (colr - i1);
  T v0[MAXM], v1[MAXM], xv[MAXM];
#pragma unroll
  for (int j = 0; j < MAXM; ++j) {
    v0[j] = (FULL || j < m) ? p0[j] : T(0);
    if (TWO) v1[j] = (FULL || j < m) ? p1[j] : T(0);
  }
#pragma unroll
  for (int j = 1; j < MAXM; ++j) xv[j] = kLazyTail<T, MAXM> ? T(0) : P.x[j] * P.h.inv;  // the reflector's tail
  T d0 = T(0), d1 = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (FULL || j < m) {
      d0 = fma_(v0[j], P.x[j], d0);
      if (TWO) d1 = fma_(v1[j], P.x[j], d1);
    }
  const T tw0 = P.h.tau * fma_(d0, P.h.inv, v0[0]);
  if (h0) {
    p0[0] = v0[0] - tw0;
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (FULL || j < m) p0[j] = fma_(-tw0, kLazyTail<T, MAXM> ? P.x[j] * P.h.inv : xv[j], v0[j]);
  }
  if (TWO && h1) {
    const T tw1 = P.h.tau * fma_(d1, P.h.inv, v1[0]);
    p1[0] = v1[0] - tw1;
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (FULL || j < m) p1[j] = fma_(-tw1, kLazyTail<T, MAXM> ? P.x[j] * P.h.inv : xv[j], v1[j]);
  }
  for (int32_t i = 129 + lane; i <= nr; i += 64) {  // bands wider than 128 rows
    int32_t si = sr + i;
    si = si >= A.W ? si - A.W : si;
    T *p = L + __umul24(si, S) + (colr - i);
    T v[MAXM];
#pragma unroll
    for (int j = 0; j < MAXM; ++j) v[j] = (FULL || j < m) ? p[j] : T(0);
    T dd = T(0);
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (FULL || j < m) dd = fma_(v[j], P.x[j], dd);
    const T tw = P.h.tau * fma_(dd, P.h.inv, v[0]);
    p[0] = v[0] - tw;
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (FULL || j < m) p[j] = fma_(-tw, kLazyTail<T, MAXM> ? P.x[j] * P.h.inv : xv[j], v[j]);
  }
}

// Column half on the ring.  Element (c+i, c+jj) sits at base[off(i) + jj],
// base = (c, c), off(i) = i*(S-1), less W*S for rows past the end of the
// ring (WRAP; rows i >= iw).
template <typename T, int MAXM, bool WRAP, int SC>
__device__ __forceinline__ void col_offsets(const Ring<T> &A, int32_t iw, int32_t (&off)[MAXM]) {
  const int32_t S = SC ? SC : A.S;
  const int32_t WS = A.W * S;
#pragma unroll
  for (int i = 0; i < MAXM; ++i) off[i] = i * (S - 1) - ((WRAP && i >= iw) ? WS : 0);
}

// Column half, first part: x = column c's entries in rows c..ch; column c
// becomes (beta, 0, ..., 0) (beta = alpha for a zero tail).
template <typename T, int MAXM, bool FULL, bool WRAP, int SC>
__device__ __forceinline__ void ring_col_prep(const Ring<T> &A, T *base, int32_t iw, int32_t m, int lane,
                                              HalfRefl<T, MAXM> &P) {
  int32_t off[MAXM];
  col_offsets<T, MAXM, WRAP, SC>(A, iw, off);
#pragma unroll
  for (int i = 0; i < MAXM; ++i) P.x[i] = (FULL || i < m) ? base[off[i]] : T(0);
  T sn = T(0);
#pragma unroll
  for (int i = 1; i < MAXM; ++i)
    if (FULL || i < m) sn = fma_(P.x[i], P.x[i], sn);
  P.h = house_from(P.x[0], sn);
  if (lane < m) {
    const int32_t S = SC ? SC : A.S;
    const int32_t o = lane * (S - 1) - ((WRAP && lane >= iw) ? A.W * S : 0);
    base[o] = lane > 0 ? T(0) : P.h.beta;
  }
}

// Column half, second part: the reflector applied from the left to columns
// c+1..jend, one lane per column (c+1+lane and, TWO, c+65+lane; wider bands
// loop).  nc = jend - c.
template <typename T, int MAXM, bool FULL, bool TWO, int SC, bool WRAP>
__device__ __forceinline__ void ring_col_apply(const Ring<T> &A, T *base, int32_t iw, int32_t m, int32_t nc,
                                               int lane, const HalfRefl<T, MAXM> &P) {
  if (!P.h.nz) return;
  int32_t off[MAXM];
  col_offsets<T, MAXM, WRAP, SC>(A, iw, off);
  const int32_t a0 = lane + 1, a1 = lane + 65;
  const bool h0 = a0 <= nc, h1 = a1 <= nc;
  T *q0 = base + (h0 ? a0 : nc), *q1 = base + (h1 ? a1 : nc);
  T v0[MAXM], v1[MAXM], xv[MAXM];
#pragma unroll
  for (int i = 0; i < MAXM; ++i) {
    v0[i] = (FULL || i < m) ? q0[off[i]] : T(0);
    if (TWO) v1[i] = (FULL || i < m) ? q1[off[i]] : T(0);
  }
#pragma unroll
  for (int i = 1; i < MAXM; ++i) xv[i] = kLazyTail<T, MAXM> ? T(0) : P.x[i] * P.h.inv;  // the reflector's tail
  T d0 = T(0), d1 = T(0);
#pragma unroll
  for (int i = 1; i < MAXM; ++i)
    if (FULL || i < m) {
      d0 = fma_(P.x[i], v0[i], d0);
      if (TWO) d1 = fma_(P.x[i], v1[i], d1);
    }
  const T tw0 = P.h.tau * fma_(d0, P.h.inv, v0[0]);
  if (h0) {
    q0[0] = v0[0] - tw0;
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) q0[off[i]] = fma_(-tw0, kLazyTail<T, MAXM> ? P.x[i] * P.h.inv : xv[i], v0[i]);
  }
  if (TWO && h1) {
    const T tw1 = P.h.tau * fma_(d1, P.h.inv, v1[0]);
    q1[0] = v1[0] - tw1;
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) q1[off[i]] = fma_(-tw1, kLazyTail<T, MAXM> ? P.x[i] * P.h.inv : xv[i], v1[i]);
  }
  for (int32_t jj = 129 + lane; jj <= nc; jj += 64) {  // bands wider than 128 columns
    T *q = base + jj;
    T v[MAXM];
#pragma unroll
    for (int i = 0; i < MAXM; ++i) v[i] = (FULL || i < m) ? q[off[i]] : T(0);
    T dd = T(0);
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) dd = fma_(P.x[i], v[i], dd);
    const T tw = P.h.tau * fma_(dd, P.h.inv, v[0]);
    q[0] = v[0] - tw;
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) q[off[i]] = fma_(-tw, kLazyTail<T, MAXM> ? P.x[i] * P.h.inv : xv[i], v[i]);
  }
}

// Wide tiles (the windowed group kernel): the defining entries live in LDS
// (xs, MAXM per sweep) instead of registers.  The first part copies them to
// xs (lane j: entry j) before the pivot overwrites them; the second part
// reads them back by broadcast.  Same arithmetic and order as the register
// versions above (x_j * inv is formed where it is used); up to 128 rows or
// columns per half (the windowed passes have at most b + t = 128).
template <typename T, int MAXM, int SC>
__device__ __forceinline__ Refl<T> ring_row_prep_x(const Ring<T> &A, int32_t sr, int32_t colr, int lane, T *xs) {
  const int32_t S = SC ? SC : A.S;
  T *px = A.L + __umul24(sr, S) + colr;
  T sn = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j) {
    const T xj = px[j];
    sn = fma_(xj, xj, sn);
  }
  const Refl<T> h = house_from(px[0], sn);
  if (lane < MAXM) {
    xs[lane] = px[lane];
    px[lane] = lane > 0 ? T(0) : h.beta;
  }
  return h;
}

template <typename T, int MAXM, bool TWO, int SC>
__device__ __forceinline__ void ring_row_apply_x(const Ring<T> &A, int32_t sr, int32_t colr, int32_t nr, int lane,
                                                 const Refl<T> &h, const T *xs) {
  if (!h.nz) return;
  const int32_t S = SC ? SC : A.S;
  T *L = A.L;
  const int32_t a0 = lane + 1, a1 = lane + 65;
  const bool h0 = a0 <= nr, h1 = a1 <= nr;
  const int32_t i0 = h0 ? a0 : nr, i1 = h1 ? a1 : nr;  // inactive lanes read row ch, store nothing
  int32_t s0 = sr + i0, s1 = sr + i1;
  s0 = s0 >= A.W ? s0 - A.W : s0;
  s1 = s1 >= A.W ? s1 - A.W : s1;
  T *p0 = L + __umul24(s0, S) + (colr - i0);
  T *p1 = L + __umul24(s1, S) + (colr - i1);
  T v0[MAXM], v1[MAXM];
#pragma unroll
  for (int j = 0; j < MAXM; ++j) {
    v0[j] = p0[j];
    if (TWO) v1[j] = p1[j];
  }
  T d0 = T(0), d1 = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j) {
    d0 = fma_(v0[j], xs[j], d0);
    if (TWO) d1 = fma_(v1[j], xs[j], d1);
  }
  const T tw0 = h.tau * fma_(d0, h.inv, v0[0]);
  if (h0) {
    p0[0] = v0[0] - tw0;
#pragma unroll
    for (int j = 1; j < MAXM; ++j) p0[j] = fma_(-tw0, xs[j] * h.inv, v0[j]);
  }
  if (TWO && h1) {
    const T tw1 = h.tau * fma_(d1, h.inv, v1[0]);
    p1[0] = v1[0] - tw1;
#pragma unroll
    for (int j = 1; j < MAXM; ++j) p1[j] = fma_(-tw1, xs[j] * h.inv, v1[j]);
  }
}

template <typename T, int MAXM, bool WRAP, int SC>
__device__ __forceinline__ Refl<T> ring_col_prep_x(const Ring<T> &A, T *base, int32_t iw, int lane, T *xs) {
  int32_t off[MAXM];
  col_offsets<T, MAXM, WRAP, SC>(A, iw, off);
  T sn = T(0);
#pragma unroll
  for (int i = 1; i < MAXM; ++i) {
    const T xi = base[off[i]];
    sn = fma_(xi, xi, sn);
  }
  const Refl<T> h = house_from(base[off[0]], sn);
  if (lane < MAXM) {
    const int32_t S = SC ? SC : A.S;
    const int32_t o = lane * (S - 1) - ((WRAP && lane >= iw) ? A.W * S : 0);
    xs[lane] = base[o];
    base[o] = lane > 0 ? T(0) : h.beta;
  }
  return h;
}

template <typename T, int MAXM, bool TWO, int SC, bool WRAP>
__device__ __forceinline__ void ring_col_apply_x(const Ring<T> &A, T *base, int32_t iw, int32_t nc, int lane,
                                                 const Refl<T> &h, const T *xs) {
  if (!h.nz) return;
  int32_t off[MAXM];
  col_offsets<T, MAXM, WRAP, SC>(A, iw, off);
  const int32_t a0 = lane + 1, a1 = lane + 65;
  const bool h0 = a0 <= nc, h1 = a1 <= nc;
  T *q0 = base + (h0 ? a0 : nc), *q1 = base + (h1 ? a1 : nc);
  T v0[MAXM], v1[MAXM];
#pragma unroll
  for (int i = 0; i < MAXM; ++i) {
    v0[i] = q0[off[i]];
    if (TWO) v1[i] = q1[off[i]];
  }
  T d0 = T(0), d1 = T(0);
#pragma unroll
  for (int i = 1; i < MAXM; ++i) {
    d0 = fma_(xs[i], v0[i], d0);
    if (TWO) d1 = fma_(xs[i], v1[i], d1);
  }
  const T tw0 = h.tau * fma_(d0, h.inv, v0[0]);
  if (h0) {
    q0[0] = v0[0] - tw0;
#pragma unroll
    for (int i = 1; i < MAXM; ++i) q0[off[i]] = fma_(-tw0, xs[i] * h.inv, v0[i]);
  }
  if (TWO && h1) {
    const T tw1 = h.tau * fma_(d1, h.inv, v1[0]);
    q1[0] = v1[0] - tw1;
#pragma unroll
    for (int i = 1; i < MAXM; ++i) q1[off[i]] = fma_(-tw1, xs[i] * h.inv, v1[i]);
  }
}

// Row half with fewer than MAXM columns where the padding columns are not
// known to be zero (tile widths below the register tile): both parts, out of
// line.
template <typename T, int MAXM, int SC>
__device__ __attribute__((noinline)) void ring_row_half_masked(const Ring<T> &A, int32_t sr, int32_t colr,
                                                               int32_t m, int32_t nr, int lane) {
  HalfRefl<T, MAXM> P;
  ring_row_prep<T, MAXM, false, SC>(A, sr, colr, m, lane, P);
  ring_row_apply<T, MAXM, false, true, SC>(A, sr, colr, m, nr, lane, P);
}

// The truncated last cycle of a sweep (m < MAXM), both parts, out of line so
// that the common path keeps its registers; its rows may also wrap around the
// ring.
template <typename T, int MAXM, int SC>
__device__ __attribute__((noinline)) void ring_col_half_rare(const Ring<T> &A, int32_t sc, int32_t m, int32_t nc,
                                                             int lane) {
  const int32_t S = SC ? SC : A.S;
  T *base = A.L + __umul24(sc, S) + A.sub;
  const int32_t iw = A.W - sc;  // rows c+i with i >= iw wrap to the start of the ring
  HalfRefl<T, MAXM> P;
  if (m == MAXM) {
    ring_col_prep<T, MAXM, true, true, SC>(A, base, iw, m, lane, P);
    if (nc > 64)
      ring_col_apply<T, MAXM, true, true, SC, true>(A, base, iw, m, nc, lane, P);
    else
      ring_col_apply<T, MAXM, true, false, SC, true>(A, base, iw, m, nc, lane, P);
  } else {
    ring_col_prep<T, MAXM, false, true, SC>(A, base, iw, m, lane, P);
    ring_col_apply<T, MAXM, false, true, SC, true>(A, base, iw, m, nc, lane, P);
  }
}

// Whether a row half takes the common path (full register tile), whose
// first part may run ahead of the waits.
template <int MAXM>
__device__ __forceinline__ bool row_common(int32_t m, int t) {
  // With an exact register tile (MAXM = t+1) a truncated last cycle
  // (m < MAXM) runs the full-width code: the entries it also reads lie past
  // column n-1 but inside the row's stored range, hold +0, leave every sum
  // and update unchanged to the bit, and get +0 written back.
  return m == MAXM || MAXM == t + 1;
}


// One sweep of the group, run by one wave.  Cycle geometry and ring slots
// advance incrementally (c by b per cycle, the slot of c likewise).
//
// Progress is published in steps: two per half-cycle done, plus one once the
// next half's first part (reflector and pivot) is done ahead of its waits.
// For b' <= 2 the second part of the predecessor's half q+d-1 touches
// nothing that this sweep's half q, or the next sweep's half q-d, touches
// (only its first part does), so half q waits for 2(q+d-1)+1 steps; for
// b' >= 3 the two second parts overlap and half q waits for 2(q+d) steps.
// Either way it waits for all 4 Kp steps once the predecessor has no half
// q+d-1 left.
//
// XL: the defining entries of the fast halves live in LDS (xs, the sweep's
// MAXM entries; wide tiles, ring_row_prep_x and the rest).
template <typename T, int MAXM, int SC, int TWO, bool XL = false>
__device__ void group_sweep(const Ring<T> &A, GroupCtl &ctl, int32_t n, int b, int t, int d, int32_t R, int j,
                            int lane, uint32_t spin_limit, uint32_t *status, uint32_t *sync, T *xs = nullptr) {
  const int32_t S = SC ? SC : A.S;
  const int32_t K = int32_t(cycles_of_dev(n, b, t, R));
  const int32_t Kp = j > 0 ? int32_t(cycles_of_dev(n, b, t, R - 1)) : 0;
  int32_t c = R + (b - t);
  int32_t sc = A.slot(c);
  int32_t known_pred = 0, known_rows = 0;
  const bool mark = b - t <= 2;                   // publish the first-part step
  const int32_t lag_steps = mark ? 2 * d - 1 : 2 * d;
  BB_P(Prof pr; pr.start();)
  // Waits before half q (rows up to `hi` resident); false: abort.
  auto wait_half = [&](int32_t q, int32_t hi) -> bool {
    if (j > 0 && !prog_wait(&ctl.sweep[j - 1], known_pred, min(2 * q + lag_steps, 4 * Kp), ctl, spin_limit, status))
      return false;
    BB_P(pr.tick(0);)
    if (!rows_wait(&ctl.loaded_hi, known_rows, hi + 1, ctl, spin_limit, status)) return false;
    BB_P(pr.tick(1);)
    return true;
  };
  // Publishes half q done; the sweep's lowest row from then on is `fl`.
  // The final count waits for the predecessor's.  False: abort.
  auto publish = [&](int32_t q, int32_t fl) -> bool {
    BB_P(pr.tick(2 + (q & 1));)
    if (q + 1 == 2 * K && j > 0 && !prog_wait(&ctl.sweep[j - 1], known_pred, 4 * Kp, ctl, spin_limit, status))
      return false;
    if (lane == 0)  // one release: the half's LDS writes are complete before either word moves
      __hip_atomic_store(&ctl.sweep[j], sweep_word(2 * (q + 1), fl), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    BB_P(pr.tick(4); pr.add(5, 1);)
    return true;
  };
  // Publishes that the first part of half q (q halves done) is done.
  auto publish_first = [&](int32_t q, int32_t fl) {
    if (mark && lane == 0)  // release: the pivot's LDS writes are complete
      __hip_atomic_store(&ctl.sweep[j], sweep_word(2 * q + 1, fl), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  for (int32_t k = 0; k < K; ++k) {
    const int32_t ch = min(c + t, n - 1);
    const int32_t m = ch - c + 1;
    const int32_t r = k == 0 ? R : c - b;
    const int32_t sr = k == 0 ? A.slot(R) : (sc - b < 0 ? sc - b + A.W : sc - b);
    const int32_t jend = min(c + t + b, n - 1);
    const int32_t nr = ch - r, colr = c - r + A.sub, nc = jend - c;
    // Row half 2k.  Its reflector comes from row r: for k > 0 the sweep's
    // previous column half left it final, so it is formed before the wait;
    // the first one (row R) may still be updated by the predecessor.
    HalfRefl<T, MAXM> Pr;
    Refl<T> hr;
    const bool row_fast = row_common<MAXM>(m, t);
    if (k > 0 && row_fast) {
      if constexpr (XL)
        hr = ring_row_prep_x<T, MAXM, SC>(A, sr, colr, lane, xs);
      else
        ring_row_prep<T, MAXM, true, SC>(A, sr, colr, MAXM, lane, Pr);
      publish_first(2 * k, r);  // the floor since the previous half: row c - b = r
    }
    if (!wait_half(2 * k, ch)) return;
    if (row_fast) {
      if constexpr (XL) {
        if (k == 0) hr = ring_row_prep_x<T, MAXM, SC>(A, sr, colr, lane, xs);
        if (TWO == 1 || (TWO == 2 && nr > 64))
          ring_row_apply_x<T, MAXM, true, SC>(A, sr, colr, nr, lane, hr, xs);
        else
          ring_row_apply_x<T, MAXM, false, SC>(A, sr, colr, nr, lane, hr, xs);
      } else {
        if (k == 0) ring_row_prep<T, MAXM, true, SC>(A, sr, colr, MAXM, lane, Pr);
        if (TWO == 1 || (TWO == 2 && nr > 64))
          ring_row_apply<T, MAXM, true, true, SC>(A, sr, colr, MAXM, nr, lane, Pr);
        else
          ring_row_apply<T, MAXM, true, false, SC>(A, sr, colr, MAXM, nr, lane, Pr);
      }
    } else {
      ring_row_half_masked<T, MAXM, SC>(A, sr, colr, m, nr, lane);
    }
    if (!publish(2 * k, c)) return;
    // Column half 2k+1: its reflector (column c, final after the row half)
    // is formed before the wait.
    HalfRefl<T, MAXM> Pc;
    T *base = A.L + __umul24(sc, S) + A.sub;
    // A full column block whose rows run past the end of the ring (rows
    // c+i, i >= iw, live at the start) takes the same path with per-row
    // offsets: about MAXM of every W slots, and every sweep of a group meets
    // it at nearly the same cycle, so it sits on the chain between sweeps.
    const bool col_fast = m == MAXM;
    const int32_t iw = A.W - sc;
    const bool col_wrap = iw < MAXM;
    Refl<T> hc;
    if (col_fast) {
      if constexpr (XL) {
        if (col_wrap)
          hc = ring_col_prep_x<T, MAXM, true, SC>(A, base, iw, lane, xs);
        else
          hc = ring_col_prep_x<T, MAXM, false, SC>(A, base, 0, lane, xs);
      } else if (col_wrap) {
        ring_col_prep<T, MAXM, true, true, SC>(A, base, iw, MAXM, lane, Pc);
      } else {
        ring_col_prep<T, MAXM, true, false, SC>(A, base, 0, MAXM, lane, Pc);
      }
      publish_first(2 * k + 1, c);
    }
    if (!wait_half(2 * k + 1, ch)) return;
    if (XL && col_fast) {
      const bool two = TWO == 1 || (TWO == 2 && nc > 64);
      if (col_wrap) {
        if (two)
          ring_col_apply_x<T, MAXM, true, SC, true>(A, base, iw, nc, lane, hc, xs);
        else
          ring_col_apply_x<T, MAXM, false, SC, true>(A, base, iw, nc, lane, hc, xs);
      } else if (two) {
        ring_col_apply_x<T, MAXM, true, SC, false>(A, base, 0, nc, lane, hc, xs);
      } else {
        ring_col_apply_x<T, MAXM, false, SC, false>(A, base, 0, nc, lane, hc, xs);
      }
    } else if (col_fast) {
      const bool two = TWO == 1 || (TWO == 2 && nc > 64);
      if (col_wrap) {
        if (two)
          ring_col_apply<T, MAXM, true, true, SC, true>(A, base, iw, MAXM, nc, lane, Pc);
        else
          ring_col_apply<T, MAXM, true, false, SC, true>(A, base, iw, MAXM, nc, lane, Pc);
      } else if (two) {
        ring_col_apply<T, MAXM, true, true, SC, false>(A, base, 0, MAXM, nc, lane, Pc);
      } else {
        ring_col_apply<T, MAXM, true, false, SC, false>(A, base, 0, MAXM, nc, lane, Pc);
      }
    } else {
      ring_col_half_rare<T, MAXM, SC>(A, sc, m, nc, lane);
    }
    if (!publish(2 * k + 1, k + 1 < K ? c : n)) return;
    c += b;
    sc += b;
    while (sc >= A.W) sc -= A.W;
  }
  BB_P(pr.flush(sync, lane);)
}

// ---- the symmetric reduction on the same ring ----------------------------
//
// The symmetric cycle (page "A two-stage reduction on an Apple M5 Pro",
// section 6; the steps and the arithmetic of bb_sym.hip) on ring rows, run
// by one wave in two half-cycles:
//   half A (rows p..c-1): the reflector from row p at columns c..ch, applied
//     to the row segments of rows p+1..c-1 (one lane each, in rounds of 64);
//     row p becomes (beta, 0, ..., 0);
//   half B (rows c..ch): the column segments of columns ch+1..min(ch+b, n-1)
//     and the symmetric block c..ch (lane i: row i of y = tau B v, then row
//     i's upper part of B -= v z^T + z v^T; the block is read in full before
//     any lane writes it, y passes between lanes through ys).
// The reflector passes from half A to half B in registers.  Ring rows are
// working-band rows: element (i, j), j >= i, at offset j - i.
template <typename T, int MAXM>
__device__ __forceinline__ void ring_seg_apply(T (&a)[MAXM], const T (&v)[MAXM], T tau, int m) {
  T s = a[0];
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (j < m) s = fma_(a[j], v[j], s);
  const T w = tau * s;
  a[0] = a[0] - w;
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (j < m) a[j] = fma_(-w, v[j], a[j]);
}

// Half A, first part: the reflector from pivot row p at columns c..ch (v in
// registers, myv = v_lane for the block), and row p becomes (beta, 0, ..., 0).
template <typename T, int MAXM>
__device__ void ring_sym_prep_a(const Ring<T> &A, int32_t c, int m, int32_t p, int lane, Refl<T> &h,
                                T (&v)[MAXM], T &myv) {
  const int32_t S = A.S;
  T *px = A.L + A.slot(p) * S + (c - p);
  T x[MAXM];
#pragma unroll
  for (int j = 0; j < MAXM; ++j) x[j] = j < m ? px[j] : T(0);
  T sn = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (j < m) sn = fma_(x[j], x[j], sn);
  h = house_from(x[0], sn);
  myv = T(0);
  if (h.nz) {
    v[0] = T(1);
#pragma unroll
    for (int j = 1; j < MAXM; ++j) v[j] = x[j] * h.inv;
    if (lane < m) myv = lane == 0 ? T(1) : px[lane] * h.inv;  // v_lane (read before the pivot write below)
  }
  if (lane < m) px[lane] = lane > 0 ? T(0) : h.beta;  // beta = alpha for a zero tail
}

// Half A, second part: the reflector applied to the row segments of rows
// p+1..c-1 at columns c..ch, one lane each, in rounds of 64.
template <typename T, int MAXM>
__device__ void ring_sym_apply_a(const Ring<T> &A, int32_t c, int m, int32_t p, int lane, const Refl<T> &h,
                                 const T (&v)[MAXM]) {
  if (!h.nz) return;
  const int32_t S = A.S;
  T *L = A.L;
  const int32_t sp = A.slot(p);
  const int32_t nr = c - p - 1;  // rows p+1..c-1 at columns c..ch
  for (int32_t q = lane; q < nr; q += 64) {
    T *pr = L + A.next(sp, 1 + q) * S + (c - (p + 1 + q));
    T a[MAXM];
#pragma unroll
    for (int j = 0; j < MAXM; ++j) a[j] = j < m ? pr[j] : T(0);
    ring_seg_apply<T, MAXM>(a, v, h.tau, m);
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j < m) pr[j] = a[j];
  }
}

template <typename T, int MAXM>
__device__ void ring_sym_half_b(const Ring<T> &A, T *ys, int32_t n, int b, int32_t c, int m, int lane,
                                const Refl<T> &h, const T (&v)[MAXM], T myv) {
  if (!h.nz) return;
  const int32_t S = A.S;
  T *L = A.L;
  const int32_t sc = A.slot(c), ch = c + m - 1;
  // y_i = tau (B(i,0) + sum_j B(i,j) v_j), B(i,j) = row c+min(i,j), offset |i-j|
  T yi = T(0);
  const int32_t si = A.next(sc, lane < m ? lane : 0);
  if (lane < m) {
    T s = L[sc * S + lane];
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (j < m) s = fma_(lane <= j ? L[si * S + (j - lane)] : L[A.next(sc, j) * S + (lane - j)], v[j], s);
    yi = h.tau * s;
    ys[lane] = yi;
  }
  const int32_t nc = min(ch + b, n - 1) - ch;  // columns ch+1.. at rows c..ch
  for (int32_t q = lane; q < nc; q += 64) {
    const int32_t col = ch + 1 + q;
    T a[MAXM];
    int32_t s = sc;
#pragma unroll
    for (int i = 0; i < MAXM; ++i) {
      if (i < m) a[i] = L[s * S + (col - c - i)];
      s = s + 1 == A.W ? 0 : s + 1;
    }
    ring_seg_apply<T, MAXM>(a, v, h.tau, m);
    s = sc;
#pragma unroll
    for (int i = 0; i < MAXM; ++i) {
      if (i < m) L[s * S + (col - c - i)] = a[i];
      s = s + 1 == A.W ? 0 : s + 1;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  T yv[MAXM];
#pragma unroll
  for (int i = 0; i < MAXM; ++i) yv[i] = i < m ? ys[i] : T(0);
  T dot = yv[0];
#pragma unroll
  for (int i = 1; i < MAXM; ++i)
    if (i < m) dot = fma_(yv[i], v[i], dot);
  const T alpha = -((T(0.5) * h.tau) * dot);
  if (lane < m) {
    const T zi = fma_(alpha, myv, yi);
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j >= lane && j < m) {
        T *e = L + si * S + (j - lane);
        *e = fma_(-myv, fma_(alpha, v[j], yv[j]), fma_(-zi, v[j], *e));
      }
  }
}

// One symmetric sweep of the group, run by one wave.  Progress is published
// in steps as for the general sweeps: two per half done, plus one once half
// A's first part (reflector and pivot) is done ahead of its wait, which for
// b' <= 2 is all the next sweep's half q needs of the predecessor's half
// q+d-1 when that is a half A; so half q waits for min(2(q+d)-1, all) steps
// of the predecessor when b' <= 2, else min(2(q+d), all), and until its rows
// are loaded; the final count waits for the predecessor's final count.
// Floors: after half A the sweep still touches rows from c, after half B
// from the next pivot row (c again).  Half A's first part runs before its
// wait for every cycle but the first: its pivot row c - b was last written
// by the sweep's own half B of the previous cycle, and no other sweep
// touches it until this half A is done.
template <typename T, int MAXM>
__device__ void sym_group_sweep(const Ring<T> &A, GroupCtl &ctl, T *ys, int32_t n, int b, int t, int d, int32_t R,
                                int j, int lane, uint32_t spin_limit, uint32_t *status) {
  const int32_t K = int32_t(cycles_of_dev(n, b, t, R));
  const int32_t Kp = j > 0 ? int32_t(cycles_of_dev(n, b, t, R - 1)) : 0;
  const bool mark = b - t <= 2;
  const int32_t lag_steps = mark ? 2 * d - 1 : 2 * d;
  int32_t known_pred = 0, known_rows = 0;
  for (int32_t k = 0; k < K; ++k) {
    const int32_t c = R + (b - t) + k * b;
    const int32_t ch = min(c + t, n - 1);
    const int m = ch - c + 1;
    const int32_t p = k == 0 ? R : c - b;
    Refl<T> h;
    T v[MAXM], myv;
    if (k > 0) {
      ring_sym_prep_a<T, MAXM>(A, c, m, p, lane, h, v, myv);
      if (mark && lane == 0)  // release: the pivot's LDS writes are complete
        __hip_atomic_store(&ctl.sweep[j], sweep_word(4 * k + 1, p), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (j > 0 && !prog_wait(&ctl.sweep[j - 1], known_pred, min(4 * k + lag_steps, 4 * Kp), ctl, spin_limit, status))
      return;
    if (!rows_wait(&ctl.loaded_hi, known_rows, c, ctl, spin_limit, status)) return;
    if (k == 0) ring_sym_prep_a<T, MAXM>(A, c, m, p, lane, h, v, myv);
    ring_sym_apply_a<T, MAXM>(A, c, m, p, lane, h, v);
    if (lane == 0)
      __hip_atomic_store(&ctl.sweep[j], sweep_word(4 * k + 2, c), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (j > 0 &&
        !prog_wait(&ctl.sweep[j - 1], known_pred, min(4 * k + 2 + lag_steps, 4 * Kp), ctl, spin_limit, status))
      return;
    if (!rows_wait(&ctl.loaded_hi, known_rows, ch + 1, ctl, spin_limit, status)) return;
    ring_sym_half_b<T, MAXM>(A, ys, n, b, c, m, lane, h, v, myv);
    if (k + 1 == K && j > 0 && !prog_wait(&ctl.sweep[j - 1], known_pred, 4 * Kp, ctl, spin_limit, status)) return;
    if (lane == 0)
      __hip_atomic_store(&ctl.sweep[j], sweep_word(4 * k + 4, k + 1 < K ? c : n), __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;



// Where ring rows come from in memory.  Whole rows (Win unused): ring row i
// is the working band's row i.  Windows: ring row i holds the bytes
// w0_bytes .. w0_bytes + ring row bytes of the band's row i (row_bytes
// apart in memory); rcp = 1 / (ring row bytes / 16), for the row of a
// chunk.
struct Win {
  int32_t row_bytes, w0_bytes;
  float rcp;
};

// c16 / rc for the 16-byte chunk c16 of windows of rc chunks (rcp = 1 / rc):
// the float quotient, corrected (c16 < 2^24).
__device__ __forceinline__ int32_t win_row(const Win &w, int32_t rc, int32_t c16) {
  int32_t i = int32_t(float(c16) * w.rcp);
  if ((i + 1) * rc <= c16) ++i;
  if (i * rc > c16) --i;
  return i;
}

// The memory offset of byte e (a multiple of 16) of ring rows lo, lo+1, ...
// stored back to back (windows of rb bytes).
__device__ __forceinline__ uint32_t win_offset(const Win &w, int32_t rb, int32_t lo, int32_t e) {
  const int32_t i = win_row(w, rb >> 4, e >> 4);
  return uint32_t((lo + i) * w.row_bytes + w.w0_bytes + (e - i * rb));
}

// A lane's walk over chunks lane, lane + 64, lane + 128, ... of ring rows
// lo, lo+1, ... stored back to back (windows of rb bytes, rc = rb / 16
// chunks each): `at` is the memory offset of the current chunk.  Moving on
// by 64 chunks is q rows and s chunks (64 = q rc + s), and one row more
// when the chunk's place in its row passes rc, so each step is a few adds
// (win_offset per chunk costs four integer multiplies).
struct WinWalk {
  int32_t r, rc, s;
  uint32_t at, d0, d1;
  WinWalk() = default;
  __device__ __forceinline__ WinWalk(const Win &w, int32_t rb, int32_t lo, int lane) {
    rc = rb >> 4;
    const int32_t q = win_row(w, rc, 64);
    s = 64 - q * rc;
    const int32_t i = win_row(w, rc, lane);
    r = lane - i * rc;
    at = uint32_t((lo + i) * w.row_bytes + w.w0_bytes + r * 16);
    d0 = uint32_t(q * w.row_bytes + s * 16);
    d1 = uint32_t(w.row_bytes - rc * 16);
  }
  __device__ __forceinline__ void step() {
    r += s;
    at += d0;
    if (r >= rc) {
      r -= rc;
      at += d1;
    }
  }
};

// Copies rows [lo, hi) of the band from memory into their ring slots with
// LDS-direct 16-byte loads (no registers involved), split where the ring
// wraps.  Complete once vmcnt reaches zero.  WIN: each ring row is a window
// of the band's row (win).
template <typename T, bool WIN = false>
__device__ void ring_fill(const Ring<T> &A, __amdgpu_buffer_rsrc_t mem, int32_t lo, int32_t hi, int lane,
                          const Win &win = Win{}) {
  const int32_t row_bytes = A.S * int32_t(sizeof(T));
  unsigned char *base = reinterpret_cast<unsigned char *>(A.L);
  while (lo < hi) {
    const int32_t s = A.slot(lo);
    const int32_t run = min(hi - lo, A.W - s);  // rows up to the end of the ring
    const int32_t bytes = run * row_bytes;
    unsigned char *dst = base + s * row_bytes;
    WinWalk wk = WIN ? WinWalk(win, row_bytes, lo, lane) : WinWalk{};
    // whole 1 KiB chunks (every lane's 16 bytes inside the run) unmasked,
    // then the last, partial one
    const int32_t whole = bytes & ~1023;
    int32_t off = 0;
#pragma unroll 4
    for (; off < whole; off += 1024) {
      const uint32_t src = WIN ? wk.at : uint32_t(lo * row_bytes + off + lane * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mem, (lds_ptr_t)(dst + off), 16, src, 0, 0, kSc1);
      if constexpr (WIN) wk.step();
    }
    if (off < bytes && off + lane * 16 < bytes) {
      const uint32_t src = WIN ? wk.at : uint32_t(lo * row_bytes + off + lane * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mem, (lds_ptr_t)(dst + off), 16, src, 0, 0, kSc1);
    }
    lo += run;
  }
}

// Writes rows [lo, hi) from their ring slots back to memory (agent-coherent
// 16-byte stores).  Complete once vmcnt reaches zero.  The LDS reads of a
// round (up to kDrainChunks 16-byte chunks per lane) are all issued before
// its stores, so the round waits for LDS once; lanes past the end of the run
// repeat its last chunk (the same bytes to the same address), so no lane is
// masked off.
constexpr int kDrainChunks = 16;
template <typename T, bool WIN = false>
__device__ void ring_drain(const Ring<T> &A, __amdgpu_buffer_rsrc_t mem, int32_t lo, int32_t hi, int lane,
                           const Win &win = Win{}) {
  const int32_t row_bytes = A.S * int32_t(sizeof(T));
  const unsigned char *base = reinterpret_cast<const unsigned char *>(A.L);
  while (lo < hi) {
    const int32_t s = A.slot(lo);
    const int32_t run = min(hi - lo, A.W - s);
    const int32_t bytes = run * row_bytes;
    const unsigned char *src = base + s * row_bytes;
    const uint32_t dst = uint32_t(lo * row_bytes);
    // windows: the walk gives each chunk's offset; lanes past the end take
    // the run's last chunk
    WinWalk wk = WIN ? WinWalk(win, row_bytes, lo, lane) : WinWalk{};
    const uint32_t last = WIN ? win_offset(win, row_bytes, lo, bytes - 16) : 0u;
    int32_t off0 = 0;
    // whole rounds: every chunk of every lane inside the run
    for (; off0 + kDrainChunks * 1024 <= bytes; off0 += kDrainChunks * 1024) {
      u32x4 v[kDrainChunks];
#pragma unroll
      for (int u = 0; u < kDrainChunks; ++u) v[u] = *reinterpret_cast<const u32x4 *>(src + off0 + u * 1024 + lane * 16);
#pragma unroll
      for (int u = 0; u < kDrainChunks; ++u) {
        __builtin_amdgcn_raw_buffer_store_b128(v[u], mem, WIN ? wk.at : dst + uint32_t(off0 + u * 1024 + lane * 16), 0,
                                               kSc1);
        if constexpr (WIN) wk.step();
      }
    }
    // the last, partial round
    if (off0 < bytes) {
      u32x4 v[kDrainChunks];
      int32_t off[kDrainChunks];
#pragma unroll
      for (int u = 0; u < kDrainChunks; ++u) {
        off[u] = min(off0 + u * 1024 + lane * 16, bytes - 16);
        v[u] = *reinterpret_cast<const u32x4 *>(src + off[u]);
      }
#pragma unroll
      for (int u = 0; u < kDrainChunks; ++u) {
        if (off0 + u * 1024 < bytes)  // wave-uniform: chunks of this round that hold any of the run
          __builtin_amdgcn_raw_buffer_store_b128(
              v[u], mem, WIN ? (off0 + u * 1024 + lane * 16 <= bytes - 16 ? wk.at : last) : dst + uint32_t(off[u]), 0,
              kSc1);
        if constexpr (WIN) wk.step();
      }
    }
    lo += run;
  }
}

// Idle accounting of the auxiliary waves: a run of empty polls is one
// bounded wait (WaitClock, restarted whenever rows move); on expiry the
// status word is set and the group aborts.  The loop that calls it reads
// the abort flag itself.
__device__ __forceinline__ bool aux_idle(WaitClock &idle, uint32_t limit, GroupCtl &ctl, uint32_t *status) {
  __builtin_amdgcn_s_sleep(1);
  if (idle.tick<256, false>(limit, status)) return true;
  lds_store(&ctl.abort_, 1);
  return false;
}

// The writer: writes back the rows every sweep is done with, up to `batch`
// rows at a time, publishing X_g = rows written after each batch.
template <typename T, bool WIN = false>
__device__ void group_writer(const Ring<T> &A, GroupCtl &ctl, __amdgpu_buffer_rsrc_t mem, int32_t n, int32_t R0,
                             int32_t Gg, uint32_t *xself_line, int lane, uint32_t spin_limit, uint32_t *status,
                             uint32_t *sync, int32_t batch, const Win &win = Win{}) {
  int32_t written = R0;
  WaitClock idle;
  for (;;) {
    // One LDS access per word, all in flight together (lane j reads sweep j's
    // word), then one acquire: the rows below every floor are then visible.
    const int32_t ab = __hip_atomic_load(&ctl.abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int32_t lh = __hip_atomic_load(&ctl.loaded_hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint64_t w = lane < Gg ? __hip_atomic_load(&ctl.sweep[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                                 : sweep_word(0, n);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (ab) return;
    const int32_t fl = sweep_floor(w);
    int32_t dead = n;
#pragma unroll
    for (int j = 0; j < kGroupMaxSweeps; ++j) dead = min(dead, __builtin_amdgcn_readlane(fl, j));
    // write back in batches, publishing after each: the next group's first
    // sweep needs the lowest released rows first
    const int32_t wb = min(min(dead, lh), written + batch);
    if (wb > written) {
      ring_drain<T, WIN>(A, mem, written, wb, lane, win);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the rows are in memory
      written = wb;
      lds_store(&ctl.written, written);  // their slots may be refilled
      if (lane == 0) __hip_atomic_store(xself_line, uint32_t(written), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      idle = WaitClock();
      if (written >= n) return;
    } else if (!aux_idle(idle, spin_limit, ctl, status)) {
      return;
    }
  }
}

// Where a group's loader learns which rows are final: the previous group's
// release counter X_{g-1} (G = 0), or, for the first group of a pass that
// follows another in the same launch, the counters of that pass's groups
// (G sweeps each, ngroups of them, the first at `line`).  Row i is touched
// by that pass's groups 0 .. q, q = min(i / G, ngroups - 1), only (a group
// touches no row below its first sweep), and X_q <= X_{q'} for q' < q, so
// X_q > i means that all of them are done with row i.  line = nullptr:
// every row is final (the launch's first pass).
struct PrevRows {
  const uint32_t *line;
  int32_t G, ngroups;
};

// The loader: polls the released rows and loads them into free ring slots,
// in batches, signalling each batch.
template <typename T, bool WIN = false>
__device__ void group_loader(const Ring<T> &A, GroupCtl &ctl, __amdgpu_buffer_rsrc_t mem, int32_t n, int32_t R0,
                             const PrevRows src, int lane, uint32_t spin_limit, uint32_t *status, uint32_t *sync,
                             const Win &win = Win{}) {
  int32_t loaded = R0;
  int32_t xprev = src.line ? 0 : n;
  WaitClock idle;
  for (;;) {
    // the three words are read together, then one acquire
    const int32_t want = min(n, loaded + kLoadBatchRows);
    if (src.G > 0) {  // the owner of the batch's last row, in the previous pass
      const int32_t q = min((want - 1) / src.G, src.ngroups - 1);
      xprev = int32_t(__hip_atomic_load(src.line + int64_t(q) * kLine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    } else if (xprev < n) {
      xprev = int32_t(__hip_atomic_load(src.line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    const int32_t ab = __hip_atomic_load(&ctl.abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int32_t wr = __hip_atomic_load(&ctl.written, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const bool failed = launch_failed(status);  // in flight with the release counter
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (ab) return;
    if (failed) {  // a wait elsewhere in the launch expired: the group drains
      lds_store(&ctl.abort_, 1);
      return;
    }
    const int32_t lim = min(min(xprev, wr + A.W), want);
    if (lim > loaded) {
      ring_fill<T, WIN>(A, mem, loaded, lim, lane, win);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the rows are in LDS
      loaded = lim;
      lds_store(&ctl.loaded_hi, loaded);
      idle = WaitClock();
      if (loaded >= n) return;
    } else if (!aux_idle(idle, spin_limit, ctl, status)) {
      return;
    }
  }
}

// Persistent group kernel: workgroups claim the groups of a run of passes
// in increasing order.  blockDim = 64 (gmax + 2); dynamic LDS = W * S *
// sizeof(T).  MAXM: the run's register tile; a pass of the run may use
// MAXM - 1 instead (variant bit 0).  SYM: the sweeps are the symmetric
// reduction's (by half-cycles, with the same lag d), every pass at MAXM.
//
// WIN (the 33-entry tile family): ring rows are windows of the band's rows
// (run.ring_stride entries from entry run.w0, every entry a pass touches),
// so that a pass of a wide working band still gets a ring of several
// sweeps; S stays the band's row stride in memory.  WIN = 1: t = 31, one row
// per lane; 2: t = 32, two rows per lane.
template <typename T, int MAXM, int SC, bool SYM = false, int WIN = 0>
__global__ void __launch_bounds__(64 * kGroupMaxWaves) k_group(T *a, int32_t S, int32_t sub, int32_t n, GroupRun run,
                                                                 int W, uint32_t *sync, uint32_t spin_limit) {
  extern __shared__ __align__(16) unsigned char lds_ring[];
  __shared__ GroupCtl ctl;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);  // wave-uniform
  const int lane = int(threadIdx.x) & 63;
  uint32_t *status = sync;
  uint32_t *claim = sync + kClaim;
  uint32_t *prog = sync + kSyncHeader;
  const Ring<T> A{reinterpret_cast<T *>(lds_ring), WIN ? run.ring_stride : S, W, WIN ? sub - run.w0 : sub};
  Win win{};
  if constexpr (WIN) {
    win.row_bytes = S * int32_t(sizeof(T));
    win.w0_bytes = run.w0 * int32_t(sizeof(T));
    win.rcp = 1.0f / float(run.ring_stride * int32_t(sizeof(T)) / 16);
  }
  const __amdgpu_buffer_rsrc_t mem =
      __builtin_amdgcn_make_buffer_rsrc(a, 0, int(uint32_t(int64_t(n) * S * int64_t(sizeof(T)))), kRsrcWord3);
  // the run's table goes to LDS once, so that no SGPRs hold it while the
  // sweeps run
  __shared__ uint32_t tab_pass[kMaxRunPasses];
  __shared__ int32_t tab_base[kMaxRunPasses];
  if (threadIdx.x == 0) {
    ctl.abort_ = 0;
#pragma unroll
    for (int j = 0; j < kMaxRunPasses; ++j) {
      tab_pass[j] = run.pass[j];
      tab_base[j] = j < run.npass ? run.base[j] : run.total;
    }
  }
  for (;;) {
    // thread 0 claims a group and looks up its pass (the last whose first
    // group is <= gi) and the pass before it in the run; the other waves
    // read them from LDS
    if (threadIdx.x == 0) {
      const int32_t gi = int32_t(atomicAdd(claim, 1u));
      uint32_t pw = tab_pass[0], qw = 0;
      int32_t base = 0, qbase = -1;
#pragma unroll
      for (int j = 1; j < kMaxRunPasses; ++j) {
        if (gi >= tab_base[j] && tab_base[j] < run.total) {
          qw = pw;
          qbase = base;
          pw = tab_pass[j];
          base = tab_base[j];
        }
      }
      if (launch_failed(status)) ctl.abort_ = 1;  // a wait elsewhere expired: drain
      ctl.g = gi;
      ctl.pass_word = pw;
      ctl.prev_word = qw;
      ctl.base = base;
      ctl.prev_base = qbase;
    }
    __syncthreads();
    const int32_t gi = __builtin_amdgcn_readfirstlane(ctl.g);  // over the run
    if (gi >= run.total || ctl.abort_) break;
    const uint32_t pw = __builtin_amdgcn_readfirstlane(ctl.pass_word);
    const int32_t base = __builtin_amdgcn_readfirstlane(ctl.base);
    const int pb = int(pw & 0x1fffu), pt = int((pw >> 13) & 0x1fffu), pG = int((pw >> 26) & 7u);
    const int variant = int(pw >> 29);
    const int pd = pb - pt >= 3 ? 2 : (pb - pt == 2 ? 3 : 4);
    const int32_t nsweeps = max(n - (pb - pt) - 1, 0);
    const int32_t g = gi - base;
    const int32_t R0 = g * pG;
    const int32_t Gg = min(pG, nsweeps - R0);
    __syncthreads();  // every wave has read the claim before thread 0 resets the control words
    if (threadIdx.x == 0) {
      ctl.loaded_hi = R0;
      ctl.written = R0;
      for (int j = 0; j < kGroupMaxSweeps; ++j) {
        ctl.sweep[j] = sweep_word(0, j < Gg ? R0 + j : n);
      }
    }
    __syncthreads();
    if (wave < Gg) {
      if constexpr (SYM) {
        __shared__ T sym_ys[kGroupMaxSweeps * MAXM];
        sym_group_sweep<T, MAXM>(A, ctl, sym_ys + wave * MAXM, n, pb, pt, pd, R0 + wave, wave, lane, spin_limit,
                                 status);
      } else {
        // the pass's tile (MAXM or MAXM - 1) and rows per lane: 1, a pass
        // with rows or columns beyond 64 per half (b + t > 64) runs the
        // two-rows-per-lane code throughout (its masks cover shorter
        // halves); 0, one row per lane; 2 (fp64, whose two-row code needs
        // twice the registers), the choice per half
        const bool lo = (variant & 1) != 0;
        const bool two = (variant & 2) != 0;
        const int32_t R = R0 + wave;
        // fp64 keeps the defining entries in LDS (their registers spill
        // otherwise); fp32 keeps them in registers, which is faster
        constexpr bool XL = sizeof(T) == 8;
        if constexpr (WIN == 2) {
          __shared__ T win_xs[XL ? kGroupMaxSweeps * MAXM : 1];
          group_sweep<T, MAXM, SC, 1, XL>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync,
                                          win_xs + (XL ? wave * MAXM : 0));
        } else if constexpr (WIN == 1) {
          __shared__ T win_xs[XL ? kGroupMaxSweeps * MAXM : 1];
          group_sweep<T, MAXM - 1, SC, 0, XL>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync,
                                              win_xs + (XL ? wave * MAXM : 0));
        } else if constexpr (sizeof(T) == 8) {
          if (lo)
            group_sweep<T, MAXM - 1, SC, 2>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
          else
            group_sweep<T, MAXM, SC, 2>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
        } else if (lo) {
          if (two)
            group_sweep<T, MAXM - 1, SC, 1>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
          else
            group_sweep<T, MAXM - 1, SC, 0>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
        } else {
          if (two)
            group_sweep<T, MAXM, SC, 1>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
          else
            group_sweep<T, MAXM, SC, 0>(A, ctl, n, pb, pt, pd, R, wave, lane, spin_limit, status, sync);
        }
      }
    } else if (wave == run.gmax) {
      group_writer<T, WIN != 0>(A, ctl, mem, n, R0, Gg, prog + int64_t(gi) * kLine, lane, spin_limit, status, sync,
                                SYM ? kDrainBatchRows : drain_batch(pb, pt), win);
    } else if (wave == run.gmax + 1) {
      PrevRows src{nullptr, 0, 0};
      if (g > 0)
        src.line = prog + int64_t(gi - 1) * kLine;
      else if (ctl.prev_base >= 0) {  // the first group of a pass after the run's first
        const uint32_t qw = ctl.prev_word;
        const int qb = int(qw & 0x1fffu), qt = int((qw >> 13) & 0x1fffu), qG = int((qw >> 26) & 7u);
        const int32_t qsweeps = max(n - (qb - qt) - 1, 0);
        src = PrevRows{prog + int64_t(ctl.prev_base) * kLine, qG, (qsweeps + qG - 1) / qG};
      }
      group_loader<T, WIN != 0>(A, ctl, mem, n, R0, src, lane, spin_limit, status, sync, win);
    }
    __syncthreads();
  }
}

template <typename T, int MAXM, int SC, int WIN = 0>
hipError_t group_t(const GroupRun &run, void *wband, const Geometry &g, int W, uint32_t *sync, int grid,
                   uint32_t spin_limit, hipStream_t st) {
  const size_t lds = size_t(W) * size_t(WIN ? run.ring_stride : g.stride) * sizeof(T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_group<T, MAXM, SC, false, WIN>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_group<T, MAXM, SC, false, WIN>), dim3(unsigned(grid)), dim3(unsigned(64 * (run.gmax + 2))),
                     lds, st, static_cast<T *>(wband), g.stride, g.sub, int32_t(g.n), run, W, sync, spin_limit);
  return hipGetLastError();
}

// Row strides with a compile-time specialisation (the working-band strides
// of BW 64 / TW 16 and BW 32 / TW 16 in fp32, BW 16 / TW 8 in fp64, BW 64 /
// TW 16 in fp16); any other stride runs the generic ring code.
template <typename T, int MAXM>
hipError_t group_stride(const GroupRun &run, void *wband, const Geometry &g, int W, uint32_t *sync, int grid,
                        uint32_t spin_limit, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {  // half precision: the headline band's stride, else the generic ring code
    if (g.stride == 104) return group_t<T, MAXM, 104>(run, wband, g, W, sync, grid, spin_limit, st);
    return group_t<T, MAXM, 0>(run, wband, g, W, sync, grid, spin_limit, st);
  } else {
    if (sizeof(T) == 4 && g.stride == 100) return group_t<T, MAXM, 100>(run, wband, g, W, sync, grid, spin_limit, st);
    if (sizeof(T) == 4 && g.stride == 68) return group_t<T, MAXM, 68>(run, wband, g, W, sync, grid, spin_limit, st);
    if (sizeof(T) == 8 && g.stride == 34) return group_t<T, MAXM, 34>(run, wband, g, W, sync, grid, spin_limit, st);
    return group_t<T, MAXM, 0>(run, wband, g, W, sync, grid, spin_limit, st);
  }
}

template <typename T>
hipError_t group_dispatch(const GroupRun &run, void *wband, const Geometry &g, int W, uint32_t *sync, int grid,
                          uint32_t spin_limit, hipStream_t st) {
  switch (run.maxm) {
    case 9: return group_stride<T, 9>(run, wband, g, W, sync, grid, spin_limit, st);
    case 17: return group_stride<T, 17>(run, wband, g, W, sync, grid, spin_limit, st);
    case 33:  // windows of wide rows, fp32 only; one pass per launch, two rows per lane: variant bit 1
      if constexpr (sizeof(T) == 4) {
        if (run.ring_stride > 0 && (run.pass[0] >> 30) & 1u)
          return group_t<T, 33, 0, 2>(run, wband, g, W, sync, grid, spin_limit, st);
        if (run.ring_stride > 0) return group_t<T, 33, 0, 1>(run, wband, g, W, sync, grid, spin_limit, st);
      }
      if constexpr (sizeof(T) == 8) {
        if (run.ring_stride > 0 && !((run.pass[0] >> 30) & 1u))
          return group_t<T, 33, 0, 1>(run, wband, g, W, sync, grid, spin_limit, st);
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MAXM>
hipError_t sym_group_t(const GroupRun &run, void *wband, const SymGeometry &g, int W, uint32_t *sync, int grid,
                       uint32_t spin_limit, hipStream_t st) {
  const size_t lds = size_t(W) * size_t(g.stride) * sizeof(T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_group<T, MAXM, 0, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_group<T, MAXM, 0, true>), dim3(unsigned(grid)), dim3(unsigned(64 * (run.gmax + 2))), lds, st,
                     static_cast<T *>(wband), g.stride, 0, int32_t(g.n), run, W, sync, spin_limit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sym_group(const GroupRun &run, void *wband, const SymGeometry &g, int W, uint32_t *sync, int grid,
                            uint32_t spin_limit, hipStream_t st) {
  if (g.dtype == 1) {
    if (run.maxm == 9) return sym_group_t<double, 9>(run, wband, g, W, sync, grid, spin_limit, st);
    if (run.maxm == 17) return sym_group_t<double, 17>(run, wband, g, W, sync, grid, spin_limit, st);
    return hipErrorInvalidValue;
  }
  if (g.dtype != 0) return hipErrorInvalidValue;
  if (run.maxm == 9) return sym_group_t<float, 9>(run, wband, g, W, sync, grid, spin_limit, st);
  if (run.maxm == 17) return sym_group_t<float, 17>(run, wband, g, W, sync, grid, spin_limit, st);
  if (run.maxm == 33) return sym_group_t<float, 33>(run, wband, g, W, sync, grid, spin_limit, st);
  return hipErrorInvalidValue;
}

hipError_t launch_group(const GroupRun &run, void *wband, const Geometry &g, int W, uint32_t *sync, int grid,
                        uint32_t spin_limit, hipStream_t st) {
  if (g.dtype == 1) return group_dispatch<double>(run, wband, g, W, sync, grid, spin_limit, st);
  if (g.dtype == 2) return group_dispatch<_Float16>(run, wband, g, W, sync, grid, spin_limit, st);
  return group_dispatch<float>(run, wband, g, W, sync, grid, spin_limit, st);
}

}  // namespace bb
