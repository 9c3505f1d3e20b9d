/*
 * Threaded runner of the CPU oracle's cycles: the all-core CPU baseline.
 * TEST INFRASTRUCTURE ONLY (like the oracle it runs).
 *
 * It executes exactly the oracle's cycle() (bb_oracle_body.h, included
 * unchanged through bb_oracle.c) but runs the sweeps of a pass on P threads,
 * the parallel schedule the pages describe (page "A two-stage reduction on an
 * Apple M5 Pro", section 6: sweep s may run a step once sweep s-1 has
 * finished the step two ahead; page "Accelerating Bidiagonalization of Banded
 * Matrices through Memory-Aware Bulge-Chasing on GPUs", three-cycle-separation
 * passage: two cycles of separation suffice when the target bandwidth
 * exceeds one, three always do).
 *
 * Thread p runs sweeps p, p+P, p+2P, ... in order.  Before cycle k of sweep R
 * it waits until sweep R-1 has completed min(k + L, K_{R-1}) cycles, L = 2
 * when b' >= 2 and 3 when b' = 1, and a sweep publishes its final count only
 * after its predecessor's final count (so "R-1 complete" implies "every
 * earlier sweep complete").  These waits imply the half-cycle rule that the
 * schedule model test proves sufficient, so the result equals the sequential
 * oracle's to the bit; the threaded tests check exactly that.  Passes are
 * separated by joining the threads.
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <sched.h>
#include <stdatomic.h>
#include <unistd.h>

#include "bb_oracle.c"

static int64_t mt_cycles_of(int64_t n, int64_t b, int64_t t, int64_t R) {
  const int64_t last = n - 2 - R - (b - t);
  return last < 0 ? 0 : last / b + 1;
}

int bb_oracle_mt_default_threads(void);

static void mt_wait(_Atomic int64_t *cnt, int64_t need) {
  int spins = 0;
  while (atomic_load_explicit(cnt, memory_order_acquire) < need)
    if (++spins > 64) {
      sched_yield();
      spins = 0;
    }
}

#define REAL double
#define SUF(name) name##_f64
#include "bb_oracle_mt_body.h"
#undef REAL
#undef SUF

#define REAL float
#define SUF(name) name##_f32
#include "bb_oracle_mt_body.h"
#undef REAL
#undef SUF

/* Threads used when nthreads <= 0: the online host cores. */
int bb_oracle_mt_default_threads(void) {
  const long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}
