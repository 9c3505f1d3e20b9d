/*
 * Body of the CPU oracle, included once per precision by bb_oracle.c with
 * REAL / FMA / SQRT / FABS / SUF defined.  TEST INFRASTRUCTURE ONLY.
 * See bb_oracle.c for what is computed and which passages it follows.
 */

/* Householder reflector for x[0..m-1] (textbook form; the page defers the
 * convention to a tile-QR paper that is not available):
 *   H = I - tau v v^T,  v = (1, x_1/(alpha-beta), ..., x_{m-1}/(alpha-beta)),
 *   beta = -sign(alpha) ||x|| (sign(+-0) = +1),  tau = (beta-alpha)/beta,
 * so that H x = beta e_1.  tau lies in [1, 2] and |v_j| <= 1, so nothing is
 * squared except inside the norm: tiny trailing entries cannot overflow or
 * divide by an underflowed zero.  Fills v[1..m-1] and returns 1, or returns
 * 0 (identity, nothing to apply) when the tail sum of squares is exactly
 * zero.  inv = 1/(alpha-beta) is returned for the dot products. */
static int SUF(house)(const REAL *x, int64_t m, REAL *beta, REAL *tau, REAL *inv, REAL *v) {
  REAL alpha = x[0];
  REAL s = 0;
  for (int64_t j = 1; j < m; ++j) s = FMA(x[j], x[j], s);
  if (s == 0) {
    *beta = alpha;
    *tau = 0;
    *inv = 0;
    return 0;
  }
  REAL nrm = SQRT(FMA(alpha, alpha, s));
  REAL bt = (alpha >= 0) ? -nrm : nrm;
  *beta = bt;
  *tau = (bt - alpha) / bt;
  *inv = (REAL)1 / (alpha - bt);
  for (int64_t j = 1; j < m; ++j) v[j] = x[j] * *inv;
  return 1;
}

/* One cycle (k) of sweep R in the pass with bandwidth b and tile width t. */
static void SUF(cycle)(REAL *a, const geom_t *gm, int64_t b, int64_t t, int64_t R, int64_t k) {
  const int64_t n = gm->n;
  const int64_t bp = b - t;
  const int64_t c = R + bp + k * b;
  if (c > n - 2) {
    fprintf(stderr, "bb_oracle: cycle (R=%lld,k=%lld) does not exist\n", (long long)R, (long long)k);
    abort();
  }
  const int64_t ch = min64(c + t, n - 1);
  const int64_t m = ch - c + 1;
  const int64_t r = (k == 0) ? R : c - b;
  REAL x[1024], v[1024];
  REAL beta, tau, inv;
  if (m > 1024) abort();

  /* 1. row reflector: annihilate A(r, c+1..ch) keeping A(r, c) */
  for (int64_t j = 0; j < m; ++j) x[j] = a[off(gm, r, c + j)];
  if (SUF(house)(x, m, &beta, &tau, &inv, v)) {
    a[off(gm, r, c)] = beta;
    for (int64_t j = 1; j < m; ++j) a[off(gm, r, c + j)] = 0;
    /* apply from the right to rows r+1..ch, columns c..ch */
    for (int64_t i = r + 1; i <= ch; ++i) {
      /* row segment A(i, c..ch): contiguous, both ends inside the band */
      REAL *p = &a[off(gm, i, c)];
      (void)off(gm, i, ch);
      /* w = A(i, c..ch) v = A(i,c) + (sum_j A(i,c+j) x_j) / (alpha-beta) */
      REAL s = 0;
      for (int64_t j = 1; j < m; ++j) s = FMA(p[j], x[j], s);
      REAL w = FMA(s, inv, p[0]);
      REAL tw = tau * w;
      p[0] = p[0] - tw;
      for (int64_t j = 1; j < m; ++j) p[j] = FMA(-tw, v[j], p[j]);
    }
  } else {
    for (int64_t j = 1; j < m; ++j) a[off(gm, r, c + j)] = 0;
  }

  /* 2. column reflector: annihilate A(c+1..ch, c) keeping A(c, c) */
  for (int64_t i = 0; i < m; ++i) x[i] = a[off(gm, c + i, c)];
  if (SUF(house)(x, m, &beta, &tau, &inv, v)) {
    a[off(gm, c, c)] = beta;
    for (int64_t i = 1; i < m; ++i) a[off(gm, c + i, c)] = 0;
    /* apply from the left to rows c..ch, columns c+1..min(c+t+b, n-1) */
    const int64_t jend = min64(c + t + b, n - 1);
    for (int64_t j = c + 1; j <= jend; ++j) {
      /* column segment A(c..ch, j): element (c+i, j) sits i*(ld-1) after
       * (c, j); both ends inside the band */
      REAL *p = &a[off(gm, c, j)];
      (void)off(gm, ch, j);
      const int64_t st = gm->ld - 1;
      /* w = v^T A(c..ch, j) = A(c,j) + (sum_i x_i A(c+i,j)) / (alpha-beta) */
      REAL s = 0;
      for (int64_t i = 1; i < m; ++i) s = FMA(x[i], p[i * st], s);
      REAL w = FMA(s, inv, p[0]);
      REAL tw = tau * w;
      p[0] = p[0] - tw;
      for (int64_t i = 1; i < m; ++i) p[i * st] = FMA(-tw, v[i], p[i * st]);
    }
  } else {
    for (int64_t i = 1; i < m; ++i) a[off(gm, c + i, c)] = 0;
  }
}

/* Copies the caller's band (row i holds A(i, i..i+bw) at band_in[i*ld_in + o])
 * into a freshly allocated working band.  Returns NULL on allocation failure. */
static REAL *SUF(load_band)(const REAL *band_in, int64_t ld_in, int bw, const geom_t *gm) {
  REAL *a = (REAL *)calloc((size_t)(gm->n * gm->ld), sizeof(REAL));
  if (!a) return NULL;
  for (int64_t i = 0; i < gm->n; ++i)
    for (int64_t o = 0; o <= bw && i + o < gm->n; ++o) a[off(gm, i, i + o)] = band_in[i * ld_in + o];
  return a;
}

static void SUF(store_out)(const REAL *a, const geom_t *gm, REAL *d, REAL *e, REAL *band_out) {
  for (int64_t i = 0; i < gm->n; ++i) {
    if (d) d[i] = a[off(gm, i, i)];
    if (e && i + 1 < gm->n) e[i] = (gm->W >= 1) ? a[off(gm, i, i + 1)] : 0;
  }
  if (band_out) memcpy(band_out, a, sizeof(REAL) * (size_t)(gm->n * gm->ld));
}

/*
 * Full reduction, passes -> sweeps -> cycles in sequential order.
 *   band_in   n rows of ld_in >= bw+1 entries (row-offset layout), read only
 *   d, e      outputs, n and n-1 entries (either may be NULL)
 *   band_out  optional copy of the final working band, n*ld entries
 *             (ld from bb_oracle_ld; element (i,j) at i*ld + j-i+T)
 *   max_cycles  stop after this many cycles (< 0: no limit); used only to
 *             time a bounded sample of a large workload
 *   cycles_done optional: number of cycles executed
 * Returns 0, or 1 on a bad argument.
 */
int SUF(bb_oracle_reduce)(const REAL *band_in, int64_t ld_in, int64_t n, int bw, int tw, REAL *d,
                          REAL *e, REAL *band_out, int64_t max_cycles, int64_t *cycles_done) {
  geom_t gm;
  if (!band_in || make_geom(n, bw, tw, &gm) || ld_in < bw + 1) return ORC_ERR_ARG;
  REAL *a = SUF(load_band)(band_in, ld_in, bw, &gm);
  if (!a) return ORC_ERR_ARG;
  int64_t done = 0;
  int stop = 0;
  for (int64_t b = bw; b > 1 && !stop; ) {
    const int64_t t = (tw < b - 1) ? tw : b - 1;
    const int64_t bp = b - t;
    for (int64_t R = 0; R + bp <= n - 2 && !stop; ++R) {
      for (int64_t k = 0; R + bp + k * b <= n - 2; ++k) {
        if (max_cycles >= 0 && done >= max_cycles) { stop = 1; break; }
        SUF(cycle)(a, &gm, b, t, R, k);
        ++done;
      }
    }
    b = bp;
  }
  SUF(store_out)(a, &gm, d, e, band_out);
  free(a);
  if (cycles_done) *cycles_done = done;
  return ORC_OK;
}

/*
 * Runs an explicit list of cycles, each a triple (pass index p, sweep R,
 * cycle k), in the order given, then writes the final working band.  Used by
 * the schedule tests: any order that respects the method's data dependences
 * must give the sequential result to the bit.  Returns 1 on a bad argument
 * or a triple that names no cycle.
 */
int SUF(bb_oracle_run_cycles)(const REAL *band_in, int64_t ld_in, int64_t n, int bw, int tw,
                              const int32_t *order, int64_t norder, REAL *band_out) {
  geom_t gm;
  if (!band_in || make_geom(n, bw, tw, &gm) || ld_in < bw + 1) return ORC_ERR_ARG;
  /* pass p has bandwidth pb[p] and tile width pt[p]; at most bw passes */
  int64_t *pb = (int64_t *)malloc(sizeof(int64_t) * (size_t)(bw + 1));
  int64_t *pt = (int64_t *)malloc(sizeof(int64_t) * (size_t)(bw + 1));
  REAL *a = SUF(load_band)(band_in, ld_in, bw, &gm);
  int rc = ORC_OK;
  int np = 0;
  if (!pb || !pt || !a) rc = ORC_ERR_ARG;
  for (int64_t b = bw; rc == ORC_OK && b > 1; ) {
    pt[np] = (tw < b - 1) ? tw : b - 1;
    pb[np] = b;
    b -= pt[np];
    ++np;
  }
  for (int64_t q = 0; rc == ORC_OK && q < norder; ++q) {
    const int32_t p = order[3 * q], R = order[3 * q + 1], k = order[3 * q + 2];
    if (p < 0 || p >= np || R < 0 || k < 0 || R + (pb[p] - pt[p]) + (int64_t)k * pb[p] > n - 2) {
      rc = ORC_ERR_ARG;
      break;
    }
    SUF(cycle)(a, &gm, pb[p], pt[p], R, k);
  }
  if (rc == ORC_OK) SUF(store_out)(a, &gm, NULL, NULL, band_out);
  free(a);
  free(pb);
  free(pt);
  return rc;
}
