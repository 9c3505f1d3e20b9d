/*
 * Band -> bidiagonal reduction by Householder bulge chasing: the CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper
 * with the HIP library; the two meet only through the seeded input generators.
 *
 * What it computes (page "Accelerating Bidiagonalization of Banded Matrices
 * through Memory-Aware Bulge-Chasing on GPUs", the three-cycle-separation
 * passage and the Algorithm 2 memory-strategy passage; page "A two-stage
 * reduction on an Apple M5 Pro", section 6):
 *
 *   An upper-banded n x n matrix A (A(i,j) != 0 only for 0 <= j-i <= BW) is
 *   reduced to upper bidiagonal form B = Q^T A P by successive band
 *   reduction.  Each pass takes the current bandwidth b to b' = b - t with
 *   t = min(TW, b-1), so the last pass lands exactly on b' = 1.
 *
 *   In a pass, sweep R (R = 0 .. n-b'-2) clears row R beyond superdiagonal
 *   b' and chases the bulge it creates down the band in cycles
 *   k = 0, 1, ... while c = R + b' + k*b <= n-2.  Each cycle annihilates one
 *   horizontal and one vertical group:
 *     1. row reflector from A(r, c..ch), r = R for k = 0 else c-b,
 *        ch = min(c+t, n-1): applied from the right to rows r+1..ch,
 *        columns c..ch; A(r,c) becomes beta, A(r,c+1..ch) exact zeros;
 *     2. column reflector from A(c..ch, c), the leftmost column of the bulge
 *        just created: applied from the left to rows c..ch, columns
 *        c+1..min(c+t+b, n-1); A(c,c) becomes beta, A(c+1..ch,c) zeros.
 *   The result is d(i) = B(i,i), e(i) = B(i,i+1).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - The reflector convention, and the treatment of near-zero entries, are
 *     deferred by the page to a tile-QR paper that is not available.  We use
 *     the textbook form H = I - tau v v^T with v = (1, x_1..x_{m-1})/(alpha -
 *     beta) past the first entry, beta = -sign(alpha) ||x|| (sign(+-0) =
 *     +1), tau = (beta - alpha)/beta.  Its scalars stay bounded (tau in
 *     [1,2], |v_j| <= 1) however small the entries, which the chase's tail
 *     needs: entries there reach 1e-23 in fp32, and a form with ||x||^2 in a
 *     denominator underflows to a division by zero.  If sum_{j>=1} x_j^2 == 0
 *     the reflector is the identity (no apply); the entries to annihilate are
 *     still written as exact zeros.
 *   - The floating-point evaluation order is fixed so that an independent
 *     implementation can reproduce results to the bit: every sum is serial in
 *     increasing index, every multiply-add is an explicit fused fma(), and
 *     nothing else is contracted (build with -ffp-contract=off).  The dot
 *     product of a row (right apply) or column (left apply) with v is
 *     s = sum_{j>=1} fma(a_j, x_j, s), w = fma(s, 1/(alpha-beta), a_0); the
 *     update is a_0 -= tau w, a_j = fma(-tau w, v_j, a_j).
 *
 * Storage: the band with room for the bulge.  Element (i,j) lives at
 * a[i*ld + (j - i + T)] for -T <= j-i <= W, with T = t of the first pass
 * (largest sub-diagonal fill) and W = BW + T (largest super-diagonal fill).
 * Every access is bounds-checked; an access outside the stored band aborts,
 * because it would mean the fill extents of the method were misread.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1

typedef struct {
  int64_t n, T, W, ld;
} geom_t;

static void die_oob(int64_t i, int64_t j, const geom_t *g) {
  fprintf(stderr,
          "bb_oracle: access (%lld,%lld) outside stored band n=%lld T=%lld W=%lld\n",
          (long long)i, (long long)j, (long long)g->n, (long long)g->T, (long long)g->W);
  abort();
}

static int64_t off(const geom_t *g, int64_t i, int64_t j) {
  if (i < 0 || j < 0 || i >= g->n || j >= g->n || j - i < -g->T || j - i > g->W)
    die_oob(i, j, g);
  return i * g->ld + (j - i + g->T);
}

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* Fills g from (n, bw, tw).  Returns 0 on success. */
static int make_geom(int64_t n, int bw, int tw, geom_t *g) {
  if (n < 1 || bw < 0 || tw < 1) return ORC_ERR_ARG;
  g->n = n;
  g->T = bw > 1 ? (tw < bw - 1 ? tw : bw - 1) : 0;
  g->W = bw + g->T;
  g->ld = g->T + g->W + 1;
  return ORC_OK;
}

/* ---- one precision at a time: the same plain code for double and float ---- */

#define REAL double
#define FMA fma
#define SQRT sqrt
#define FABS fabs
#define SUF(name) name##_f64
#include "bb_oracle_body.h"
#undef REAL
#undef FMA
#undef SQRT
#undef FABS
#undef SUF

#define REAL float
#define FMA fmaf
#define SQRT sqrtf
#define FABS fabsf
#define SUF(name) name##_f32
#include "bb_oracle_body.h"
#undef REAL
#undef FMA
#undef SQRT
#undef FABS
#undef SUF

/* Number of stored diagonals of the oracle's working band (for exports). */
int64_t bb_oracle_ld(int64_t n, int bw, int tw) {
  geom_t g;
  if (make_geom(n, bw, tw, &g)) return -1;
  return g.ld;
}

/* Sub-diagonals stored below the main diagonal in an export (T). */
int64_t bb_oracle_T(int64_t n, int bw, int tw) {
  geom_t g;
  if (make_geom(n, bw, tw, &g)) return -1;
  return g.T;
}
