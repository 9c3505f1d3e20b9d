/*
 * Symmetric band -> tridiagonal reduction by Householder bulge chasing: the
 * CPU ORACLE of the symmetric variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes (page "A two-stage reduction on an Apple M5 Pro",
 * section 6: the band chase, with LAPACK's symmetric-band kernels for the
 * symmetric case; a sweep clears one row and chases its bulge down the band a
 * block of b at a time, one reflector per step):
 *
 *   A symmetric n x n matrix of bandwidth BW (A(i,j) = 0 for |i-j| > BW) is
 *   reduced to tridiagonal form T = Q^T A Q.  As for the general band, each
 *   pass takes the bandwidth b to b' = b - t, t = min(TW, b-1), so the last
 *   pass lands on b' = 1; TW >= BW-1 is the one-pass reduction.
 *
 *   In a pass, sweep R (R = 0 .. n-b'-2) clears row R beyond superdiagonal
 *   b' and chases the bulge down the band in cycles k = 0, 1, ... while
 *   c = R + b' + k*b <= n-2.  Cycle k, with p = R for k = 0 else c-b,
 *   ch = min(c+t, n-1), S = {c..ch}:
 *     - reflector H from the row segment A(p, c..ch): A(p,c) becomes beta,
 *       A(p,c+1..ch) exact zeros (and the symmetric column);
 *     - A <- H A H on the rest: rows p+1..c-1 at columns S from the right,
 *       the symmetric block S x S from both sides, and columns
 *       ch+1..min(ch+b, n-1) at rows S from the left.  No other entry of
 *       A(., S) is nonzero at that point.
 *   Fill reaches b+t superdiagonals.  The result is d(i) = T(i,i),
 *   e(i) = T(i,i+1).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - the reflector as in the general-band oracle (bb_oracle.c):
 *     beta = -sign(alpha)||x||, tau = (beta-alpha)/beta, v = (1, x_1..)/(alpha-beta),
 *     identity when the tail is exactly zero (entries still written as zeros);
 *   - v_j = x_j * inv is formed once (rounded);
 *   - one-sided apply to a segment a (a row at columns S, or a column at
 *     rows S): s = a_0, s = fma(a_j, v_j, s) for j = 1.. in order, w = tau*s,
 *     a_0 = a_0 - w, a_j = fma(-w, v_j, a_j);
 *   - two-sided apply to the symmetric block B (the form of LAPACK's
 *     symmetric rank-2 reflector update): y_i = tau * (sum_j B(i,j) v_j,
 *     serial in j, starting from B(i,0)), dot = sum_i y_i v_i (serial, from
 *     y_0), alpha = -((tau/2) * dot), z_i = fma(alpha, v_i, y_i),
 *     B(i,j) = fma(-v_i, z_j, fma(-z_i, v_j, B(i,j))) for i <= j;
 *   - nothing else is contracted (build with -ffp-contract=off).
 *
 * Storage: the upper triangle of the band with room for the fill.  Element
 * (i,j), 0 <= j-i <= W = BW + T (T = t of the first pass), lives at
 * a[i*ld + (j - i)], ld = W + 1.  Every access is bounds-checked and aborts
 * outside the stored band.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1

typedef struct {
  int64_t n, W, ld;
} sgeom_t;

static void sdie(int64_t i, int64_t j, const sgeom_t *g) {
  fprintf(stderr, "bb_oracle_sym: access (%lld,%lld) outside stored band n=%lld W=%lld\n", (long long)i,
          (long long)j, (long long)g->n, (long long)g->W);
  abort();
}

static int64_t soff(const sgeom_t *g, int64_t i, int64_t j) {
  if (i < 0 || j < 0 || i >= g->n || j >= g->n || j - i < 0 || j - i > g->W) sdie(i, j, g);
  return i * g->ld + (j - i);
}

static int64_t smin64(int64_t a, int64_t b) { return a < b ? a : b; }

static int make_sgeom(int64_t n, int bw, int tw, sgeom_t *g) {
  if (n < 1 || bw < 0 || tw < 1) return 1;
  const int64_t T = bw >= 2 ? (tw < bw - 1 ? tw : bw - 1) : 0;
  g->n = n;
  g->W = bw + T;
  g->ld = g->W + 1;
  return 0;
}

/* Stored superdiagonals of the working band (W+1). */
int64_t bb_oracle_sym_ld(int64_t n, int bw, int tw) {
  sgeom_t g;
  return make_sgeom(n, bw, tw, &g) ? -1 : g.ld;
}

#define REAL double
#define SUF(name) name##_f64
#include "bb_oracle_sym_body.h"
#undef REAL
#undef SUF

#define REAL float
#define SUF(name) name##_f32
#include "bb_oracle_sym_body.h"
#undef REAL
#undef SUF
