// HIP kernels (gfx950) of the band -> bidiagonal reduction.
//
// One cycle of a sweep (page "Accelerating Bidiagonalization of Banded
// Matrices through Memory-Aware Bulge-Chasing on GPUs", Algorithm 2
// passage): the t+1 entries of the row to annihilate are staged in LDS, every
// thread forms the Householder reflector from them, then each thread owns one
// row of the right-apply block (t+1 entries in VGPRs), applies the reflector
// and writes the row back; the same is repeated for the leftmost column of
// the bulge just created, one thread per column of the left-apply block.
//
// The arithmetic contract the kernels follow is stated in bb_device.hpp.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_device.hpp"
#include "bb_internal.hpp"

namespace bb {
namespace {

// Vector access to the m <= MAXM consecutive entries of one band row segment
// (16-byte loads/stores where they fit, a scalar tail otherwise).  A
// full-width load may run past the segment: those values are never used, and
// anything past the end of the band reads as zero (buffer bounds).

template <typename T, int MAXM, class B>
__device__ __forceinline__ void load_seg(const B &A, uint32_t o, T (&v)[MAXM]) {
  constexpr int PER = 16 / int(sizeof(T));  // elements per 16-byte access
#ifdef BB_SCALAR_SEG
  constexpr int NV = 0;
#else
  constexpr int NV = MAXM / PER;
#endif
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    // Reinterpret the whole 16-byte vector at once: per-component casts of
    // the load builtin's result let the compiler shrink it to one dword.
    typedef T vecT __attribute__((ext_vector_type(PER)));
    const vecT x = __builtin_bit_cast(vecT, A.ld4_(o + uint32_t(q * 16)));
#pragma unroll
    for (int j = 0; j < PER; ++j) v[PER * q + j] = x[j];
  }
#pragma unroll
  for (int j = NV * PER; j < MAXM; ++j) v[j] = A.ld_(o + uint32_t(j * sizeof(T)));
}

template <typename T, int MAXM, bool FULL, class B>
__device__ __forceinline__ void store_seg(const B &A, uint32_t o, const T (&v)[MAXM], int m) {
  constexpr int PER = 16 / int(sizeof(T));
#ifdef BB_SCALAR_SEG
  constexpr int NV = 0;
#else
  constexpr int NV = MAXM / PER;
#endif
  if (FULL) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      typedef T vecT __attribute__((ext_vector_type(PER)));
      vecT y;
#pragma unroll
      for (int j = 0; j < PER; ++j) y[j] = v[PER * q + j];
      const u32x4 x = __builtin_bit_cast(u32x4, y);
      A.st4_(o + uint32_t(q * 16), x);
    }
#pragma unroll
    for (int j = NV * PER; j < MAXM; ++j) A.st_(o + uint32_t(j * sizeof(T)), v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j < m) A.st_(o + uint32_t(j * sizeof(T)), v[j]);
  }
}

// What a half does once its early part is stored (see k_persist): nothing
// for the schedulers whose halves are ordered by launches or barriers.
// kOnePass: the column half updates and stores each column in one pass
// instead of updating every column first and storing in two groups.
// Measured on the headline band: the barrier kernel wants the one pass
// (947 against 1171 ms: the two phases cost it scalar registers and a wave
// per SIMD), the step kernel the two phases (586 against 617 ms).
struct NoPub {
  static constexpr bool kOnePass = true;
  __device__ __forceinline__ void operator()() const {}
};
struct NoPubTwoPhase {
  static constexpr bool kOnePass = false;
  __device__ __forceinline__ void operator()() const {}
};

// Row half of a cycle, executed by the whole workgroup: one band row per
// thread, rows r..ch, each row's m entries (columns c..ch) loaded straight
// into VGPRs with vector loads.  Row r is the reflector input: its thread
// stages it in LDS (xs); every thread then forms the reflector and the
// threads of rows r+1..ch apply it from the right.  Row r becomes (beta,
// 0, ..., 0); column c of rows c..ch goes to LDS (ys) for the column half.
// The whole half is its early part: pub runs after every store.
template <typename T, int MAXM, bool FULL, class B, class Pub>
__device__ void row_half(const B &A, const Cyc &q, T *xs, T *ys, const Pub &pub) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int m = q.m;
  const int nr = int(q.ch - q.r) + 1;
  const uint32_t rstep = A.row_step();
  const uint32_t o0 = A.off(q.r, q.c);
  T v[MAXM];
  if (tid < nr) load_seg<T, MAXM>(A, o0 + uint32_t(tid) * rstep, v);
  if (tid == 0) {
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (FULL || j < m) xs[j] = v[j];
  }
  __syncthreads();
  const Refl<T> h = house<T, MAXM, FULL>(xs, m);
  for (int i = tid; i < nr; i += nt) {
    const uint32_t o = o0 + uint32_t(i) * rstep;
    if (i != tid) load_seg<T, MAXM>(A, o, v);  // rows beyond the workgroup
    if (i == 0) {
      if (h.nz) v[0] = h.beta;
#pragma unroll
      for (int j = 1; j < MAXM; ++j) v[j] = T(0);
    } else if (h.nz) {
      T s = T(0);
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (FULL || j < m) s = fma_(v[j], xs[j], s);
      const T w = fma_(s, h.inv, v[0]);
      const T tw = h.tau * w;
      v[0] = v[0] - tw;
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (FULL || j < m) v[j] = fma_(-tw, xs[j] * h.inv, v[j]);
    }
    const int ic = i - int(q.c - q.r);  // row c + ic
    if (ic >= 0) ys[ic] = v[0];
    if (i == 0 || h.nz) store_seg<T, MAXM, FULL>(A, o, v, m);
  }
  pub();
}

// Column half: one band column per thread, columns c..jend, each column's m
// entries (rows c..ch, (ld-1) elements apart) loaded into VGPRs; threads of
// consecutive columns touch consecutive words.  The reflector comes from the
// updated column c in LDS (ys); columns c+1..jend are updated from the left
// and column c becomes (beta, 0, ..., 0).  Columns c..c+early (the early
// part) are done first, then pub runs, then the rest.
template <typename T, int MAXM, bool FULL, class B, class Pub>
__device__ void col_half(const B &A, const Cyc &q, const T *ys, int early, const Pub &pub) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int m = q.m;
  const int nc = int(q.jend - q.c) + 1;
  const uint32_t rstep = A.row_step();
  const uint32_t o0 = A.off(q.c, q.c);
  // The thread's first column: tid, except that thread 0 (column c is the
  // pivot's, stored by every thread below) takes column nt when the
  // two-phase half has exactly nt + 1 columns, so that such a band costs no
  // second round of loads (with more columns the round is needed anyway,
  // and thread 0's far column would only spread its wave's first loads).
  // Thread tid goes on with first + nt, first + 2 nt, ...
  const int first = (tid >= 1 || Pub::kOnePass || nc != nt + 1) ? tid : nt;
  T v[MAXM];
  if (first >= 1 && first < nc) {
#pragma unroll
    for (int i = 0; i < MAXM; ++i) v[i] = A.ld_(o0 + uint32_t(first) * uint32_t(sizeof(T)) + uint32_t(i) * rstep);
  }
  const Refl<T> g = house<T, MAXM, FULL>(ys, m);
  if constexpr (Pub::kOnePass) {
    for (int jj = tid; jj < nc; jj += nt) {
      const uint32_t o = o0 + uint32_t(jj) * uint32_t(sizeof(T));
      if (jj == 0) {
        A.st_(o, g.nz ? g.beta : ys[0]);
        for (int i = 1; i < m; ++i) A.st_(o + uint32_t(i) * rstep, T(0));
        continue;
      }
      if (!g.nz) continue;
      if (jj != tid) {
#pragma unroll
        for (int i = 0; i < MAXM; ++i) v[i] = A.ld_(o + uint32_t(i) * rstep);
      }
      T s = T(0);
#pragma unroll
      for (int i = 1; i < MAXM; ++i)
        if (FULL || i < m) s = fma_(ys[i], v[i], s);
      const T w = fma_(s, g.inv, v[0]);
      const T tw = g.tau * w;
      A.st_(o, v[0] - tw);
#pragma unroll
      for (int i = 1; i < MAXM; ++i)
        if (FULL || i < m) A.st_(o + uint32_t(i) * rstep, fma_(-tw, ys[i] * g.inv, v[i]));
    }
    return;
  }
  // column jj's updated entries into v (v holds its old ones)
  auto update = [&](int jj) {
    T s = T(0);
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) s = fma_(ys[i], v[i], s);
    const T w = fma_(s, g.inv, v[0]);
    const T tw = g.tau * w;
    v[0] = v[0] - tw;
#pragma unroll
    for (int i = 1; i < MAXM; ++i)
      if (FULL || i < m) v[i] = fma_(-tw, ys[i] * g.inv, v[i]);
  };
  auto store = [&](int jj) {
    const uint32_t o = o0 + uint32_t(jj) * uint32_t(sizeof(T));
#pragma unroll
    for (int i = 0; i < MAXM; ++i)
      if (FULL || i < m) A.st_(o + uint32_t(i) * rstep, v[i]);
  };
  auto beyond = [&]() {  // columns past the workgroup's first nt
    if (!g.nz) return;
    for (int jj = first + nt; jj < nc; jj += nt) {
      const uint32_t o = o0 + uint32_t(jj) * uint32_t(sizeof(T));
#pragma unroll
      for (int i = 0; i < MAXM; ++i) v[i] = A.ld_(o + uint32_t(i) * rstep);
      update(jj);
      store(jj);
    }
  };
  // A workgroup of at most early threads may hold early columns past its
  // first nt: it finishes the half before publishing.  Otherwise the early
  // columns 1..early are first columns of threads 1..early.
  const bool split = nt > early;
  // the thread's first column: updated, and stored now if early
  const bool own = first >= 1 && first < nc && g.nz;
  if (own) update(first);
  // column c becomes (beta, 0, ..., 0): thread tid writes entries tid,
  // tid + nt, ... (m may exceed nt), so that no one thread stores the whole
  // column one entry at a time
  for (int i = tid; i < m; i += nt) A.st_(o0 + uint32_t(i) * rstep, i > 0 ? T(0) : (g.nz ? g.beta : ys[0]));
  if (own && (first <= early || !split)) store(first);
  if (!split) {
    beyond();
    pub();
    return;
  }
  pub();
  if (own && first > early) store(first);
  beyond();
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// 16-byte chunks that cover MAXM consecutive entries from any element-aligned
// start: one staged row of the block.
template <typename T, int MAXM>
constexpr int stage_chunks() {
  return (MAXM * int(sizeof(T)) + 16 - int(sizeof(T)) + 15) / 16;
}

// Row half with the block staged in LDS (persistent kernel, wide tiles whose
// block fits): the workgroup first copies the 16-byte chunks covering rows
// r..ch, columns c..ch from memory straight into LDS (LDS-direct loads,
// consecutive chunks on consecutive lanes, so one load instruction reads a
// few whole lines instead of one piece of 64 different rows).  Each thread
// then takes its row from LDS, applies the reflector formed from row r in
// LDS and puts the row back; the block is then stored element by element
// (consecutive lanes, consecutive addresses).  Arithmetic, operation order
// and results are those of row_half.
//
// Rows r+1..r+early (the early part) are stored first, then pub runs, then
// the rest.
template <typename T, int MAXM, bool FULL, int AUX, class Pub>
__device__ void row_half_staged(const Band<T, AUX> &A, const Cyc &q, unsigned char *blk, T *ys, int early,
                                const Pub &pub) {
  constexpr int CH = stage_chunks<T, MAXM>();
  constexpr int RB = CH * 16;  // LDS bytes per staged row
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int lane = tid & 63;
  const int m = FULL ? MAXM : q.m;
  const int nr = int(q.ch - q.r) + 1;
  const uint32_t rstep = A.row_step();
  const uint32_t o0 = A.off(q.r, q.c);
  const int nch = nr * CH;
  {
    // thread tid copies chunks tid, tid + nt, ...: chunk cc of row ci,
    // stepped with adds (nt = qc CH + sc); whole waves of chunks unmasked,
    // then the last, partial one
    const int qc = nt / CH, sc = nt - qc * CH;
    int ci = tid / CH, cc = tid - ci * CH;
    uint32_t srow = o0 + uint32_t(ci) * rstep;
    const uint32_t dsrow = uint32_t(qc) * rstep;
    int e0 = tid - lane;
    for (; e0 + 64 <= nch; e0 += nt) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(A.r, (lds_ptr_t)(blk + e0 * 16), 16,
                                               (srow & ~15u) + uint32_t(cc) * 16u, 0, 0, AUX);
      cc += sc;
      srow += dsrow;
      if (cc >= CH) {
        cc -= CH;
        srow += rstep;
      }
    }
    if (e0 < nch && e0 + lane < nch)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(A.r, (lds_ptr_t)(blk + e0 * 16), 16,
                                               (srow & ~15u) + uint32_t(cc) * 16u, 0, 0, AUX);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  const T *x0 = reinterpret_cast<const T *>(blk + (o0 & 15u));  // row r, columns c..ch
  const Refl<T> h = house<T, MAXM, FULL>(x0, m);
  T v[MAXM];
  for (int i = tid; i < nr; i += nt) {
    const uint32_t o = o0 + uint32_t(i) * rstep;
    T *row = reinterpret_cast<T *>(blk + i * RB + (o & 15u));
#pragma unroll
    for (int j = 0; j < MAXM; ++j) v[j] = (FULL || j < m) ? row[j] : T(0);
    if (i == 0) {
      if (h.nz) v[0] = h.beta;
#pragma unroll
      for (int j = 1; j < MAXM; ++j) v[j] = T(0);
    } else if (h.nz) {
      T s = T(0);
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (FULL || j < m) s = fma_(v[j], x0[j], s);
      const T w = fma_(s, h.inv, v[0]);
      const T tw = h.tau * w;
      v[0] = v[0] - tw;
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (FULL || j < m) v[j] = fma_(-tw, x0[j] * h.inv, v[j]);
    }
    const int ic = i - int(q.c - q.r);  // row c + ic
    if (ic >= 0) ys[ic] = v[0];
    if (i == 0) {
      store_seg<T, MAXM, FULL>(A, o, v, m);  // row r: (beta, 0, ..., 0); others still read it in LDS
    } else if (h.nz) {
#pragma unroll
      for (int j = 0; j < MAXM; ++j)
        if (FULL || j < m) row[j] = v[j];
    }
  }
  if (!h.nz) {  // uniform: every thread formed the same reflector; rows r+1..ch unchanged
    pub();
    return;
  }
  __syncthreads();
  // rows r+1..ch, element by element: consecutive lanes store consecutive
  // entries of a row.  Thread tid takes elements e = tid, tid + nt, ...
  // (row 1 + e / m, entry e % m), stepping row and entry with adds only
  // (nt = qs m + ss), eight at a time so that one LDS wait covers eight
  // reads.  The rest continues the same walk after the publish: every
  // element at or past ep is on some thread's walk from there.
  const int ne = (nr - 1) * m;
  const int ep = min(early, nr - 1) * m;
  const int qs = nt / m, ss = nt - qs * m;
  const int i0 = 1 + tid / m;
  int e = tid, j = tid - (i0 - 1) * m;
  uint32_t ro = o0 + uint32_t(i0) * rstep;  // element (i, 0) in memory
  int lr = i0 * RB;                          // staged row i in LDS
  const uint32_t dro = uint32_t(qs) * rstep;
  const int dlr = qs * RB;
  auto step = [&]() {
    e += nt;
    j += ss;
    ro += dro;
    lr += dlr;
    if (j >= m) {
      j -= m;
      ro += rstep;
      lr += RB;
    }
  };
  auto run = [&](int lim) {
    while (e + 7 * nt < lim) {
      uint32_t g[8];
      T v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        g[u] = ro + uint32_t(j * int(sizeof(T)));
        v[u] = reinterpret_cast<const T *>(blk + lr + (ro & 15u))[j];
        step();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) A.st_(g[u], v[u]);
    }
    for (; e < lim; step()) A.st_(ro + uint32_t(j * int(sizeof(T))), reinterpret_cast<const T *>(blk + lr + (ro & 15u))[j]);
  };
  run(ep);
  pub();
  run(ne);
}

template <typename T, int MAXM, int AUX, class Pub>
__device__ __forceinline__ void row_half_staged_any(const Band<T, AUX> &A, const Cyc &q, unsigned char *blk, T *ys,
                                                    int early, const Pub &pub) {
  if (q.m == MAXM)
    row_half_staged<T, MAXM, true, AUX>(A, q, blk, ys, early, pub);
  else
    row_half_staged<T, MAXM, false, AUX>(A, q, blk, ys, early, pub);
}

template <typename T, int MAXM, class B, class Pub = NoPub>
__device__ __forceinline__ void row_half_any(const B &A, const Cyc &q, T *xs, T *ys, const Pub &pub = Pub()) {
  if (q.m == MAXM)
    row_half<T, MAXM, true>(A, q, xs, ys, pub);
  else
    row_half<T, MAXM, false>(A, q, xs, ys, pub);
}

template <typename T, int MAXM, class B, class Pub = NoPub>
__device__ __forceinline__ void col_half_any(const B &A, const Cyc &q, const T *ys, int early = 0,
                                             const Pub &pub = Pub()) {
  if (q.m == MAXM)
    col_half<T, MAXM, true>(A, q, ys, early, pub);
  else
    col_half<T, MAXM, false>(A, q, ys, early, pub);
}

// One launch per step L of a pass: block q runs sweep R = Rlo + q, cycle
// k = L - s R (page: Algorithm 1, one kernel launch per cycle, kernel
// completion as the synchronisation).
template <typename T, int MAXM>
__global__ void __launch_bounds__(256) k_step(T *a, int64_t ld, int32_t sub, int64_t n, int b, int t, int64_t L,
                                              int s, int64_t Rlo) {
  __shared__ T xs[MAXM];
  __shared__ T ys[MAXM];
  const Band<T, 0> A = make_band<T, 0>(a, ld, sub, n);
  const int64_t R = Rlo + blockIdx.x;
  const Cyc q(n, b, t, R, L - int64_t(s) * R);
  row_half_any<T, MAXM>(A, q, xs, ys);
  // the column half reloads cells the row half just stored
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  col_half_any<T, MAXM>(A, q, ys, 0, NoPubTwoPhase());
}


// Progress of sweep R-1 that half h of cycle k of sweep R waits for, in
// steps: half-cycle p (2k: row half, 2k+1: column half) done counts 2p + 2,
// and 2p + 1 once every earlier half is done and half p's early part -- its
// pivot and the t + 1 rows (row half) or columns (column half) after it --
// is stored (persist_early may make the early part the whole half).  Half
// p = 2k + h needs sweep R-1's halves before p + d - 1 done and the early
// part of half p + d - 1, with d = 2 when b' >= 3, 3 when
// b' = 2 and 4 when b' = 1 (the page's rule: two cycles of separation only
// when the target band is wider than bidiagonal): no cell of this half lies
// in the rest of that half or in any later one.  Capped at all of R-1; the
// cap is only sound because a sweep publishes its final count after its
// predecessor has published its own: "sweep R-1 complete" then implies
// "every earlier sweep complete", which the truncated windows at the last
// column need (there sweeps further back than R-1 still overlap).
__device__ __forceinline__ int64_t steps_needed(int b, int t, int64_t k, int h, int64_t kprev) {
  const int bp = b - t;
  const int d = bp >= 3 ? 2 : (bp == 2 ? 3 : 4);
  const int64_t all = 4 * kprev;
  const int64_t need = 2 * (2 * k + h + d - 1) + 1;
  return need < all ? need : all;
}

// Bounded poll of a progress counter (one thread).  Returns false, with the
// status word set, once the wait expires (WaitClock: `limit` ticks, or any
// other wait of the launch expired).
__device__ __forceinline__ bool wait_progress(const uint32_t *line, uint32_t need, uint32_t limit,
                                              uint32_t *status) {
  WaitClock wc;
  while (__hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
    __builtin_amdgcn_s_sleep(1);
    if (!wc.tick(limit, status)) return false;
  }
  return true;
}

// Rows or columns after the pivot that a persistent half stores and
// publishes before the rest (k_persist): t + 1, the least the successor
// needs; b + t + 1, the whole half.  A sweep trails its predecessor by about
// (d - 1) half periods plus the part of a half before its publish, so the
// early publish pays where d = 2 (b' >= 3).  Where d >= 3 it pays only if
// the half's period does not grow: measured (d = 4), fp32 halves keep their
// period and gain, fp64 ones (heavier register pressure) grow by about 10%
// and lose, so fp64 publishes those halves whole.
template <typename T>
__host__ __device__ __forceinline__ int persist_early(int b, int t) {
  return (b - t >= 3 || sizeof(T) != 8) ? t + 1 : b + t + 1;
}

// Publishes `step` on a sweep's progress line once every store issued so
// far by the workgroup is complete (whole workgroup; see k_persist).
template <int AUX>
struct PersistPub {
  static constexpr bool kOnePass = false;
  uint32_t *line;
  uint32_t step;
  __device__ __forceinline__ void operator()() const {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
      if (AUX == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(line, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

// Persistent scheduler: each workgroup claims sweeps in increasing order
// (an atomic counter), and runs all cycles of its sweep; before each half
// cycle it waits on its predecessor's progress counter (steps_needed).  A
// half stores its early part first and publishes it (step 2p + 1) before
// it stores the rest, so the successor, which needs nothing else of that
// half, starts while the rest is still being stored; the rest is complete
// before the sweep's next half reads anything (every wave waits for its
// stores, then the workgroup meets) and before any later publish.  Claims
// are monotone, so every sweep waited on is held by a
// running workgroup: no deadlock for any grid size.  Waits are bounded by
// time (WaitClock); on expiry the workgroup sets the status word and stops,
// and every other workgroup stops at its next wait or claim.
//
// STAGED: row halves go through row_half_staged (the block in LDS, coalesced
// copies) instead of row_half (one row per lane straight to VGPRs).
//
// AUX selects how band data crosses between workgroups (and XCDs, whose L2
// caches are not coherent with each other): kSc1 makes every band access an
// agent-coherent one, so completing the stores (vmcnt 0) before the counter
// moves is the whole release; 0 uses ordinary cached accesses with an
// agent-scope release fence (L2 write-back) before each publish and an
// acquire fence (invalidate) after each wait.
#ifndef BB_PERSIST_AUX
#define BB_PERSIST_AUX 16
#endif
template <typename T, int MAXM, int AUX, bool STAGED>
__global__ void __launch_bounds__(256) k_persist(T *a, int64_t ld, int32_t sub, int64_t n, int b, int t,
                                                 int64_t nsweeps, uint32_t *sync, uint32_t spin_limit) {
  const Band<T, AUX> A = make_band<T, AUX>(a, ld, sub, n);
  __shared__ T xs[MAXM];
  __shared__ T ys[MAXM];
  extern __shared__ __attribute__((aligned(16))) unsigned char blk[];  // staged block (row halves)
  __shared__ int64_t sR;
  __shared__ int sgo;
  uint32_t *status = sync;
  uint32_t *claim = sync + kClaim;
  uint32_t *prog = sync + kSyncHeader;
  const int tid = threadIdx.x;
  const int early = persist_early<T>(b, t);
#ifdef BB_PROFILE
  // wall-clock ticks spent waiting, in row halves, column halves, publishing
  uint64_t t_wait = 0, t_row = 0, t_col = 0, t_pub = 0, n_half = 0, t_mark = 0;
  unsigned long long *prof = reinterpret_cast<unsigned long long *>(sync + kProf);
#define BB_TICK(acc)                        \
  do {                                      \
    const uint64_t now_ = wall_clock64();   \
    acc += now_ - t_mark;                   \
    t_mark = now_;                          \
  } while (0)
#else
#define BB_TICK(acc) \
  do {               \
  } while (0)
#endif
  if (tid == 0) sgo = 1;
  for (;;) {
    if (tid == 0) {
      sR = int64_t(atomicAdd(claim, 1u));
      if (launch_failed(status)) sgo = 0;  // a wait elsewhere expired: drain
    }
    __syncthreads();
    const int64_t R = sR;
    if (R >= nsweeps || !sgo) break;
    const int64_t K = cycles_of_dev(A.n, b, t, R);
    const int64_t Kp = R > 0 ? cycles_of_dev(A.n, b, t, R - 1) : 0;
    const uint32_t *pred = prog + (R - 1) * kLine;
    uint32_t *mine = prog + R * kLine;
    for (int64_t k = 0; k < K; ++k) {
      const Cyc q(A.n, b, t, R, k);
      for (int h = 0; h < 2; ++h) {
#ifdef BB_PROFILE
        t_mark = wall_clock64();
        ++n_half;
#endif
        if (R > 0 && tid == 0) {
          sgo = wait_progress(pred, uint32_t(steps_needed(b, t, k, h, Kp)), spin_limit, status);
          if (AUX == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        // the previous half's late stores complete (every wave), then the
        // workgroup meets: this half may read what they wrote
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (!sgo) return;
        BB_TICK(t_wait);
        const PersistPub<AUX> pub{mine, uint32_t(2 * (2 * k + h) + 1)};
        if (h == 0) {
          if constexpr (STAGED)
            row_half_staged_any<T, MAXM, AUX>(A, q, blk, ys, early, pub);
          else
            row_half_any<T, MAXM>(A, q, xs, ys, pub);
          BB_TICK(t_row);
        } else {
          col_half_any<T, MAXM>(A, q, ys, early, pub);
          BB_TICK(t_col);
        }
      }
    }
    // The final count: every store complete, and only after the
    // predecessor's final count.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      const bool go = R == 0 || wait_progress(pred, uint32_t(4 * Kp), spin_limit, status);
      if (AUX == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (go)
        __hip_atomic_store(mine, uint32_t(4 * K), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        sgo = 0;  // the final count never moves: successors time out in turn
    }
    BB_TICK(t_pub);
    __syncthreads();  // sR is rewritten by the next claim
  }
#ifdef BB_PROFILE
  if (tid == 0) {
    atomicAdd(prof + 0, (unsigned long long)t_wait);
    atomicAdd(prof + 1, (unsigned long long)t_row);
    atomicAdd(prof + 2, (unsigned long long)t_col);
    atomicAdd(prof + 3, (unsigned long long)t_pub);
    atomicAdd(prof + 4, (unsigned long long)n_half);
  }
#endif
#undef BB_TICK
}

// Grid-barrier scheduler: one launch per pass with every workgroup resident
// (one per CU).  Step L of the step scheduler -- every sweep R with cycle
// k = L - s R in range -- is shared out among the workgroups, and all of them
// meet at a device-wide barrier before step L + 1 (the page's Algorithm 1
// schedule with the kernel boundary replaced by a barrier inside one
// launch).  Band accesses are agent-coherent (sc1): a workgroup's stores are
// complete (vmcnt 0) before it arrives, so the barrier orders the steps as
// the kernel boundary does.  The barrier wait is bounded (WaitClock); on
// expiry the status word is set and every workgroup leaves at its next
// barrier.
template <typename T, int MAXM>
__global__ void __launch_bounds__(256) k_barrier(T *a, int64_t ld, int32_t sub, int64_t n, int b, int t, int s,
                                                 int64_t nsweeps, int64_t steps, uint32_t *sync,
                                                 uint32_t spin_limit) {
  const Band<T, kSc1> A = make_band<T, kSc1>(a, ld, sub, n);
  __shared__ T xs[MAXM];
  __shared__ T ys[MAXM];
  __shared__ int sgo;
  uint32_t *status = sync;
  uint32_t *arrived = sync + kClaim;  // arrivals at the current barrier
  uint32_t *gen = sync + kSyncHeader;  // barrier generation, a line of its own
  const int tid = threadIdx.x;
  const int64_t bp = b - t;
  for (int64_t L = 0; L < steps; ++L) {
    // sweeps with 0 <= L - s R < K_R
    const int64_t rhi = L / s < nsweeps - 1 ? L / s : nsweeps - 1;
    const int64_t num = L * b - (n - 2 - bp), den = int64_t(s) * b - 1;
    const int64_t rlo = num <= 0 ? 0 : (num + den - 1) / den;
    for (int64_t R = rlo + blockIdx.x; R <= rhi; R += gridDim.x) {
      const Cyc q(n, b, t, R, L - int64_t(s) * R);
      row_half_any<T, MAXM>(A, q, xs, ys);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the column half reloads cells the row half stored
      __syncthreads();
      col_half_any<T, MAXM>(A, q, ys);
      __syncthreads();  // xs, ys are reused by the next cycle
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (tid == 0) {
      // read the generation before arriving: it cannot move without us
      const uint32_t g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bool go = true;
      if (atomicAdd(arrived, 1u) == gridDim.x - 1) {
        __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(gen, g0 + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        WaitClock wc;
        while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
          __builtin_amdgcn_s_sleep(1);
          if (!wc.tick(spin_limit, status)) {
            go = false;
            break;
          }
        }
      }
      sgo = go && !launch_failed(status);
    }
    __syncthreads();
    if (!sgo) return;
  }
}

// User band (row-offset layout) -> working band with zeroed bulge room.
template <typename T>
__global__ void k_pack(const T *__restrict__ band, int64_t ld_band, int64_t n, int bw, T *__restrict__ a,
                       int64_t stride, int sub) {
  const int64_t total = n * stride;
  for (int64_t q = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; q < total;
       q += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i = q / stride;
    const int64_t o = q - i * stride - sub;  // j - i
    T v = T(0);
    if (o >= 0 && o <= bw && i + o < n) v = band[i * ld_band + o];
    a[q] = v;
  }
}

template <typename T>
__global__ void k_extract(const T *__restrict__ a, int64_t stride, int sub, int64_t n, T *__restrict__ d,
                          T *__restrict__ e) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    d[i] = a[i * stride + sub];
    // stride >= sub + 2 always (padding to 16 bytes); with bw = 0 the entry is padding and reads zero
    if (e != nullptr && i + 1 < n) e[i] = a[i * stride + sub + 1];
  }
}

__global__ void k_fill_u32(uint32_t *p, int64_t count, uint32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

inline unsigned grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return unsigned(g);
}

template <typename T, int MAXM>
hipError_t step_t(void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo, int64_t nblk,
                  int nt, hipStream_t st) {
  hipLaunchKernelGGL((k_step<T, MAXM>), dim3(unsigned(nblk)), dim3(nt), 0, st,
                     static_cast<T *>(wband),
                     int64_t(g.stride), g.sub, g.n, b, t, L, s, Rlo);
  return hipGetLastError();
}

template <typename T>
hipError_t step_dispatch(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                         int64_t nblk, int nt, hipStream_t st) {
  switch (maxm) {
    case 8: return step_t<T, 8>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 9: return step_t<T, 9>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 16: return step_t<T, 16>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 17: return step_t<T, 17>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 32: return step_t<T, 32>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 33: return step_t<T, 33>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 64: return step_t<T, 64>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 65: return step_t<T, 65>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    default: return hipErrorInvalidValue;
  }
}

// LDS for the staged row half: the block's rows (at most b + t + 1) of
// stage_chunks 16-byte chunks.  Staging pays for wide tiles (t + 1 >= 32)
// on blocks of at least kStageMinBytes (measured: the unstaged half's
// per-lane row accesses, one row per lane, cost 2-5x the staged copies once
// every CU is busy; the smallest wide block, 64 x 32 fp32, still gains with
// 128 threads); other blocks, and blocks above kStageLdsBytes, take the
// unstaged row half.
#ifndef BB_PERSIST_STAGE
#define BB_PERSIST_STAGE 1
#endif
constexpr size_t kStageLdsBytes = 64 * 1024;
constexpr size_t kStageMinBytes = 8 * 1024;

template <typename T, int MAXM>
bool staged_t(int b, int t) {
  const size_t lds = size_t(b + t + 1) * size_t(stage_chunks<T, MAXM>()) * 16;
  const size_t block = size_t(b + t + 1) * size_t(MAXM) * sizeof(T);
  return BB_PERSIST_STAGE && MAXM >= 32 && block >= kStageMinBytes && lds <= kStageLdsBytes;
}

template <typename T, int MAXM>
hipError_t barrier_t(void *wband, const Geometry &g, int b, int t, int s, int64_t nsweeps, int64_t steps,
                     uint32_t *sync, int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  hipLaunchKernelGGL((k_barrier<T, MAXM>), dim3(unsigned(grid)), dim3(nt), 0, st, static_cast<T *>(wband),
                     int64_t(g.stride), g.sub, g.n, b, t, s, nsweeps, steps, sync, spin_limit);
  return hipGetLastError();
}

template <typename T>
hipError_t barrier_dispatch(int maxm, void *wband, const Geometry &g, int b, int t, int s, int64_t nsweeps,
                            int64_t steps, uint32_t *sync, int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  switch (maxm) {
    case 8: return barrier_t<T, 8>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 9: return barrier_t<T, 9>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 16: return barrier_t<T, 16>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 17: return barrier_t<T, 17>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 32: return barrier_t<T, 32>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 33: return barrier_t<T, 33>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 64: return barrier_t<T, 64>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    case 65: return barrier_t<T, 65>(wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MAXM>
hipError_t persist_t(void *wband, const Geometry &g, int b, int t, int64_t nsweeps, uint32_t *sync, int grid,
                     int nt, uint32_t spin_limit, hipStream_t st) {
  const size_t lds = size_t(b + t + 1) * size_t(stage_chunks<T, MAXM>()) * 16;
  if (staged_t<T, MAXM>(b, t))
    hipLaunchKernelGGL((k_persist<T, MAXM, BB_PERSIST_AUX, true>), dim3(unsigned(grid)), dim3(nt), lds, st,
                       static_cast<T *>(wband), int64_t(g.stride), g.sub, g.n, b, t, nsweeps, sync, spin_limit);
  else
    hipLaunchKernelGGL((k_persist<T, MAXM, BB_PERSIST_AUX, false>), dim3(unsigned(grid)), dim3(nt), 0, st,
                       static_cast<T *>(wband), int64_t(g.stride), g.sub, g.n, b, t, nsweeps, sync, spin_limit);
  return hipGetLastError();
}

template <typename T>
hipError_t persist_dispatch(int maxm, void *wband, const Geometry &g, int b, int t, int64_t nsweeps, uint32_t *sync,
                            int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  switch (maxm) {
    case 8: return persist_t<T, 8>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 9: return persist_t<T, 9>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 16: return persist_t<T, 16>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 17: return persist_t<T, 17>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 32: return persist_t<T, 32>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 33: return persist_t<T, 33>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 64: return persist_t<T, 64>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 65: return persist_t<T, 65>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t stage_lds_bytes(int dtype, int maxm, int b, int t) {
  (void)b;
  (void)t;
  return size_t(2 * maxm) * (dtype == 1 ? 8 : (dtype == 2 ? 2 : 4));
}

template <typename T>
bool staged_dispatch(int maxm, int b, int t) {
  switch (maxm) {
    case 32: return staged_t<T, 32>(b, t);
    case 33: return staged_t<T, 33>(b, t);
    case 64: return staged_t<T, 64>(b, t);
    case 65: return staged_t<T, 65>(b, t);
    default: return false;
  }
}

bool persist_staged(int dtype, int maxm, int b, int t) {
  if (dtype == 1) return staged_dispatch<double>(maxm, b, t);
  if (dtype == 2) return staged_dispatch<_Float16>(maxm, b, t);
  return staged_dispatch<float>(maxm, b, t);
}

hipError_t launch_barrier(int maxm, void *wband, const Geometry &g, int b, int t, int s, int64_t nsweeps,
                          int64_t steps, uint32_t *sync, int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  if (g.dtype == 1)
    return barrier_dispatch<double>(maxm, wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
  if (g.dtype == 2) return hipErrorInvalidValue;  // no fp16 instantiation (as the step kernel)
  return barrier_dispatch<float>(maxm, wband, g, b, t, s, nsweeps, steps, sync, grid, nt, spin_limit, st);
}

hipError_t launch_persist(int maxm, void *wband, const Geometry &g, int b, int t, int64_t nsweeps, uint32_t *sync,
                          int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  if (g.dtype == 1) return persist_dispatch<double>(maxm, wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
  if (g.dtype == 2)
    return persist_dispatch<_Float16>(maxm, wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
  return persist_dispatch<float>(maxm, wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
}

hipError_t launch_pack(const void *band, int64_t ld_band, void *wband, const Geometry &g, hipStream_t st) {
  const int block = 256;
  const unsigned grid = grid_for(g.n * g.stride, block);
  if (g.dtype == 1)
    hipLaunchKernelGGL(k_pack<double>, dim3(grid), dim3(block), 0, st, static_cast<const double *>(band), ld_band,
                       g.n, g.bw, static_cast<double *>(wband), int64_t(g.stride), g.sub);
  else if (g.dtype == 2)
    hipLaunchKernelGGL(k_pack<_Float16>, dim3(grid), dim3(block), 0, st, static_cast<const _Float16 *>(band),
                       ld_band, g.n, g.bw, static_cast<_Float16 *>(wband), int64_t(g.stride), g.sub);
  else
    hipLaunchKernelGGL(k_pack<float>, dim3(grid), dim3(block), 0, st, static_cast<const float *>(band), ld_band,
                       g.n, g.bw, static_cast<float *>(wband), int64_t(g.stride), g.sub);
  return hipGetLastError();
}

hipError_t launch_extract(const void *wband, const Geometry &g, void *d, void *e, hipStream_t st) {
  const int block = 256;
  const unsigned grid = grid_for(g.n, block);
  if (g.dtype == 1)
    hipLaunchKernelGGL(k_extract<double>, dim3(grid), dim3(block), 0, st, static_cast<const double *>(wband),
                       int64_t(g.stride), g.sub, g.n, static_cast<double *>(d), static_cast<double *>(e));
  else if (g.dtype == 2)
    hipLaunchKernelGGL(k_extract<_Float16>, dim3(grid), dim3(block), 0, st, static_cast<const _Float16 *>(wband),
                       int64_t(g.stride), g.sub, g.n, static_cast<_Float16 *>(d), static_cast<_Float16 *>(e));
  else
    hipLaunchKernelGGL(k_extract<float>, dim3(grid), dim3(block), 0, st, static_cast<const float *>(wband),
                       int64_t(g.stride), g.sub, g.n, static_cast<float *>(d), static_cast<float *>(e));
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, int64_t count, uint32_t v, hipStream_t st) {
  const int block = 256;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(count, block)), dim3(block), 0, st, p, count, v);
  return hipGetLastError();
}

hipError_t launch_step(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                       int64_t nblk, int nt, hipStream_t st) {
  if (g.dtype == 1) return step_dispatch<double>(maxm, wband, g, b, t, L, s, Rlo, nblk, nt, st);
  if (g.dtype == 2) return hipErrorInvalidValue;  // fp16 runs on the persistent scheduler only
  return step_dispatch<float>(maxm, wband, g, b, t, L, s, Rlo, nblk, nt, st);
}

}  // namespace bb
