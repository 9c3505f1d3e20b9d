/*
 * Singular values of an upper bidiagonal matrix by bisection: the CPU ORACLE
 * of the step that follows the band -> bidiagonal reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the bench's CPU
 * baseline may load this library.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes (page "A two-stage reduction on an Apple M5 Pro",
 * section 7): the singular values of B (diagonal d_0..d_{n-1}, superdiagonal
 * e_0..e_{n-2}) are the non-negative eigenvalues of the 2n x 2n Golub-Kahan
 * tridiagonal T: zero diagonal, off-diagonal b_1..b_{2n-1} = d_0, e_0, d_1,
 * e_1, ..., d_{n-1}.  Every eigenvalue is found on its own: start from T's
 * Gershgorin interval and halve it a fixed number of times, keeping the half
 * that holds the eigenvalue by a Sturm count (the number of eigenvalues of T
 * that are <= x, read off the signs of the pivots of T - xI = LDL^T) with
 * LAPACK's guard against tiny pivots.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *   - Sturm count at x: q_1 = -x; q_j = -(bb_{j-1} / q_{j-1}) - x for
 *     j = 2..2n, bb_j = b_j * b_j (rounded products); whenever |q_j| < pivmin
 *     it is replaced by -pivmin; the count is the number of q_j <= 0.  This is
 *     LAPACK's pivot recurrence with a zero diagonal.
 *   - pivmin = m_min * max(1, max_j bb_j), m_min the smallest normal number
 *     of the precision (LAPACK's choice: pivots stay far from overflow).
 *   - Interval: r = max_i (|b_{i-1}| + |b_i|) over the rows of T (the
 *     Gershgorin radius; every centre is 0), widened for rounding by
 *     delta = ((r * 2n) * eps) + 2 * pivmin, eps the machine epsilon
 *     (2^-23 or 2^-52): [lo, hi] = [-(r + delta), r + delta].
 *   - Halvings: p + 2 of them, p the precision's significand bits (26 fp32,
 *     55 fp64), which takes the interval below half an ulp of r.  Each takes
 *     mid = 0.5 * (lo + hi) and keeps [lo, mid] when count(mid) >= j (the
 *     eigenvalue's ascending 1-based index), else [mid, hi].
 *   - Result: 0.5 * (lo + hi) of the final interval; a result that is not
 *     positive (a singular value of zero, to the bisection's resolution)
 *     is returned as +0.
 *   - Order: sigma_0 >= sigma_1 >= ...; sigma_i is eigenvalue 2n - i of T.
 * All arithmetic is in the precision of d and e, each operation rounded on
 * its own (build with -ffp-contract=off).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1

#define REAL double
#define SUF(name) name##_f64
#define REAL_MIN DBL_MIN
#define REAL_EPS DBL_EPSILON
#define REAL_HALVINGS (DBL_MANT_DIG + 2)
#include "bb_oracle_svals_body.h"
#undef REAL
#undef SUF
#undef REAL_MIN
#undef REAL_EPS
#undef REAL_HALVINGS

#define REAL float
#define SUF(name) name##_f32
#define REAL_MIN FLT_MIN
#define REAL_EPS FLT_EPSILON
#define REAL_HALVINGS (FLT_MANT_DIG + 2)
#include "bb_oracle_svals_body.h"
#undef REAL
#undef SUF
#undef REAL_MIN
#undef REAL_EPS
#undef REAL_HALVINGS
