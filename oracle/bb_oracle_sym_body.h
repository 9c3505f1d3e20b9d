/*
 * Body of the symmetric oracle, included once per precision by
 * bb_oracle_sym.c with REAL and SUF defined.  TEST INFRASTRUCTURE ONLY.
 */

#define SFMA(a, b, c) ((sizeof(REAL) == sizeof(float)) ? (REAL)fmaf((float)(a), (float)(b), (float)(c)) \
                                                       : (REAL)fma((double)(a), (double)(b), (double)(c)))
#define SSQRT(a) ((sizeof(REAL) == sizeof(float)) ? (REAL)sqrtf((float)(a)) : (REAL)sqrt((double)(a)))

/* Reflector of x[0..m-1]: returns 0 for the identity (tail exactly zero). */
static int SUF(shouse)(const REAL *x, int64_t m, REAL *beta, REAL *tau, REAL *inv) {
  const REAL alpha = x[0];
  REAL s = 0;
  for (int64_t j = 1; j < m; ++j) s = SFMA(x[j], x[j], s);
  if (s == 0) return 0;
  const REAL nrm = SSQRT(SFMA(alpha, alpha, s));
  const REAL bt = (alpha >= 0) ? -nrm : nrm;
  *beta = bt;
  *tau = (bt - alpha) / bt;
  *inv = (REAL)1 / (alpha - bt);
  return 1;
}

/* One-sided apply of H = I - tau v v^T (v_0 = 1) to a[0..m-1] (stride st). */
static void SUF(sapply)(REAL *a, int64_t st, const REAL *v, int64_t m, REAL tau) {
  REAL s = a[0];
  for (int64_t j = 1; j < m; ++j) s = SFMA(a[j * st], v[j], s);
  const REAL w = tau * s;
  a[0] = a[0] - w;
  for (int64_t j = 1; j < m; ++j) a[j * st] = SFMA(-w, v[j], a[j * st]);
}

static void SUF(scycle)(REAL *a, const sgeom_t *gm, int64_t b, int64_t t, int64_t R, int64_t k) {
  const int64_t n = gm->n;
  const int64_t c = R + (b - t) + k * b;
  const int64_t ch = smin64(c + t, n - 1);
  const int64_t m = ch - c + 1;
  const int64_t p = (k == 0) ? R : c - b;
  REAL x[m], v[m], y[m], z[m];
  for (int64_t j = 0; j < m; ++j) x[j] = a[soff(gm, p, c + j)];
  REAL beta = 0, tau = 0, inv = 0;
  if (SUF(shouse)(x, m, &beta, &tau, &inv)) {
    v[0] = 1;
    for (int64_t j = 1; j < m; ++j) v[j] = x[j] * inv;
    /* rows p+1 .. c-1 at columns S, from the right */
    for (int64_t i = p + 1; i < c; ++i) {
      REAL *row = &a[soff(gm, i, c)];
      (void)soff(gm, i, ch);
      SUF(sapply)(row, 1, v, m, tau);
    }
    /* columns ch+1 .. min(ch+b, n-1) at rows S, from the left */
    for (int64_t j = ch + 1; j <= smin64(ch + b, n - 1); ++j) {
      REAL *col = &a[soff(gm, c, j)];
      (void)soff(gm, ch, j);
      SUF(sapply)(col, gm->ld - 1, v, m, tau);
    }
    /* symmetric block S x S from both sides */
    for (int64_t i = 0; i < m; ++i) {
      REAL s = a[soff(gm, c, c + i)]; /* B(i,0) = B(0,i) */
      for (int64_t j = 1; j < m; ++j) {
        const REAL bij = (i <= j) ? a[soff(gm, c + i, c + j)] : a[soff(gm, c + j, c + i)];
        s = SFMA(bij, v[j], s);
      }
      y[i] = tau * s;
    }
    REAL dot = y[0];
    for (int64_t i = 1; i < m; ++i) dot = SFMA(y[i], v[i], dot);
    const REAL alpha = -(((REAL)0.5 * tau) * dot);
    for (int64_t i = 0; i < m; ++i) z[i] = SFMA(alpha, v[i], y[i]);
    for (int64_t i = 0; i < m; ++i)
      for (int64_t j = i; j < m; ++j) {
        REAL *e = &a[soff(gm, c + i, c + j)];
        *e = SFMA(-v[i], z[j], SFMA(-z[i], v[j], *e));
      }
    a[soff(gm, p, c)] = beta;
  }
  for (int64_t j = 1; j < m; ++j) a[soff(gm, p, c + j)] = 0;
}

static REAL *SUF(sload_band)(const REAL *band_in, int64_t ld_in, int bw, const sgeom_t *gm) {
  REAL *a = (REAL *)calloc((size_t)(gm->n * gm->ld), sizeof(REAL));
  if (!a) return NULL;
  for (int64_t i = 0; i < gm->n; ++i)
    for (int64_t o = 0; o <= bw && i + o < gm->n; ++o) a[soff(gm, i, i + o)] = band_in[i * ld_in + o];
  return a;
}

static void SUF(sstore_out)(const REAL *a, const sgeom_t *gm, REAL *d, REAL *e, REAL *band_out) {
  for (int64_t i = 0; i < gm->n; ++i) {
    if (d) d[i] = a[soff(gm, i, i)];
    if (e && i + 1 < gm->n) e[i] = gm->W >= 1 ? a[soff(gm, i, i + 1)] : 0;
  }
  if (band_out) memcpy(band_out, a, sizeof(REAL) * (size_t)(gm->n * gm->ld));
}

/*
 * Reduces the symmetric band given by its upper rows: band_in row i (stride
 * ld_in >= bw+1) holds A(i, i..i+bw), entries past n ignored.  d: n, e: n-1
 * (may be NULL when n == 1), band_out (optional): n * ld working band.
 * Returns 0, or 1 on a bad argument.
 */
int SUF(bb_oracle_sym_reduce)(const REAL *band_in, int64_t ld_in, int64_t n, int bw, int tw, REAL *d, REAL *e,
                              REAL *band_out) {
  sgeom_t gm;
  if (!band_in || make_sgeom(n, bw, tw, &gm) || ld_in < bw + 1) return ORC_ERR_ARG;
  REAL *a = SUF(sload_band)(band_in, ld_in, bw, &gm);
  if (!a) return ORC_ERR_ARG;
  for (int64_t b = bw; b > 1;) {
    const int64_t t = (tw < b - 1) ? tw : b - 1;
    const int64_t bp = b - t;
    for (int64_t R = 0; R + bp <= n - 2; ++R)
      for (int64_t k = 0; R + bp + k * b <= n - 2; ++k) SUF(scycle)(a, &gm, b, t, R, k);
    b = bp;
  }
  SUF(sstore_out)(a, &gm, d, e, band_out);
  free(a);
  return ORC_OK;
}

/*
 * Runs the listed cycles (pass, R, k) in the given order (schedule tests)
 * and returns the working band.  Returns 1 on a bad argument or an entry
 * that is not a cycle of the reduction.
 */
int SUF(bb_oracle_sym_run_cycles)(const REAL *band_in, int64_t ld_in, int64_t n, int bw, int tw,
                                  const int32_t *order, int64_t norder, REAL *band_out) {
  sgeom_t gm;
  if (!band_in || !band_out || make_sgeom(n, bw, tw, &gm) || ld_in < bw + 1) return ORC_ERR_ARG;
  REAL *a = SUF(sload_band)(band_in, ld_in, bw, &gm);
  if (!a) return ORC_ERR_ARG;
  int64_t pb[64], pt[64];
  int np = 0;
  for (int64_t b = bw; b > 1 && np < 64; ++np) {
    pt[np] = (tw < b - 1) ? tw : b - 1;
    pb[np] = b;
    b -= pt[np];
  }
  int rc = ORC_OK;
  for (int64_t q = 0; q < norder && rc == ORC_OK; ++q) {
    const int32_t ps = order[3 * q], R = order[3 * q + 1], k = order[3 * q + 2];
    if (ps < 0 || ps >= np || R < 0 || k < 0 || R + (pb[ps] - pt[ps]) + (int64_t)k * pb[ps] > n - 2) {
      rc = ORC_ERR_ARG;
      break;
    }
    SUF(scycle)(a, &gm, pb[ps], pt[ps], R, k);
  }
  if (rc == ORC_OK) SUF(sstore_out)(a, &gm, NULL, NULL, band_out);
  free(a);
  return rc;
}

#undef SFMA
#undef SSQRT
