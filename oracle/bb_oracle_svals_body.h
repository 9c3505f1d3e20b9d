/*
 * Body of the bisection oracle, included once per precision by
 * bb_oracle_svals.c with REAL, SUF, REAL_MIN, REAL_EPS and REAL_HALVINGS
 * defined.  TEST INFRASTRUCTURE ONLY.
 */

/* Off-diagonal entry j (1-based, 1..2n-1) of the Golub-Kahan tridiagonal. */
static REAL SUF(gk_b)(const REAL *d, const REAL *e, int64_t n, int64_t j) {
  if (j < 1 || j > 2 * n - 1) abort();
  return (j % 2 == 1) ? d[(j - 1) / 2] : e[j / 2 - 1];
}

/* Number of eigenvalues of the Golub-Kahan tridiagonal that are <= x. */
int64_t SUF(bb_oracle_gk_count)(const REAL *d, const REAL *e, int64_t n, REAL x, REAL pivmin) {
  int64_t count = 0;
  REAL q = -x;
  for (int64_t j = 1; j <= 2 * n; ++j) {
    if (j > 1) {
      const REAL b = SUF(gk_b)(d, e, n, j - 1);
      q = -((b * b) / q) - x;
    }
    if (fabs(q) < pivmin) q = -pivmin;
    if (q <= 0) ++count;
  }
  return count;
}

/* pivmin, and the widened Gershgorin interval [lo, hi] of the tridiagonal. */
void SUF(bb_oracle_gk_interval)(const REAL *d, const REAL *e, int64_t n, REAL *lo, REAL *hi,
                                REAL *pivmin) {
  REAL bbmax = 0, r = 0;
  for (int64_t j = 1; j <= 2 * n - 1; ++j) {
    const REAL b = SUF(gk_b)(d, e, n, j);
    if (b * b > bbmax) bbmax = b * b;
  }
  for (int64_t i = 1; i <= 2 * n; ++i) {   /* row i of T: neighbours b_{i-1}, b_i */
    const REAL left = i > 1 ? fabs(SUF(gk_b)(d, e, n, i - 1)) : 0;
    const REAL right = i < 2 * n ? fabs(SUF(gk_b)(d, e, n, i)) : 0;
    if (left + right > r) r = left + right;
  }
  const REAL pm = REAL_MIN * (bbmax > 1 ? bbmax : 1);
  const REAL delta = ((r * (REAL)(2 * n)) * REAL_EPS) + 2 * pm;
  *lo = -(r + delta);
  *hi = r + delta;
  *pivmin = pm;
}

/*
 * sigma[i - i0] = singular value i (descending, 0-based) of B for
 * i0 <= i < i1.  d has n entries, e n-1 (may be NULL when n == 1).
 * Returns 0, or 1 on a bad argument.
 */
int SUF(bb_oracle_svals)(const REAL *d, const REAL *e, int64_t n, int64_t i0, int64_t i1, REAL *sigma) {
  if (n < 0 || i0 < 0 || i1 < i0 || i1 > n) return ORC_ERR_ARG;
  if (n == 0 || i1 == i0) return ORC_OK;
  if (!d || !sigma || (n > 1 && !e)) return ORC_ERR_ARG;
  REAL lo0, hi0, pivmin;
  SUF(bb_oracle_gk_interval)(d, e, n, &lo0, &hi0, &pivmin);
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t j = 2 * n - i;
    REAL lo = lo0, hi = hi0;
    for (int h = 0; h < REAL_HALVINGS; ++h) {
      const REAL mid = (REAL)0.5 * (lo + hi);
      if (SUF(bb_oracle_gk_count)(d, e, n, mid, pivmin) >= j)
        hi = mid;
      else
        lo = mid;
    }
    const REAL s = (REAL)0.5 * (lo + hi);
    sigma[i - i0] = s > 0 ? s : 0;
  }
  return ORC_OK;
}
