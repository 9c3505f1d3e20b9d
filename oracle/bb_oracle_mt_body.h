/*
 * Body of the threaded runner, included once per precision by
 * bb_oracle_mt.c with REAL / SUF defined.  TEST INFRASTRUCTURE ONLY.
 */

typedef struct {
  REAL *a;
  const geom_t *gm;
  int64_t b, t, ns;
  int64_t lag;  /* L: cycles of separation */
  int nthreads, id;
  _Atomic int64_t *done; /* cycles completed, per sweep */
} SUF(mt_job_t);

static void *SUF(mt_worker)(void *arg) {
  const SUF(mt_job_t) *j = (const SUF(mt_job_t) *)arg;
  const int64_t n = j->gm->n;
  for (int64_t R = j->id; R < j->ns; R += j->nthreads) {
    const int64_t K = mt_cycles_of(n, j->b, j->t, R);
    const int64_t Kp = R > 0 ? mt_cycles_of(n, j->b, j->t, R - 1) : 0;
    for (int64_t k = 0; k < K; ++k) {
      if (R > 0) mt_wait(&j->done[R - 1], min64(k + j->lag, Kp));
      SUF(cycle)(j->a, j->gm, j->b, j->t, R, k);
      if (k == K - 1 && R > 0) mt_wait(&j->done[R - 1], Kp);
      atomic_store_explicit(&j->done[R], k + 1, memory_order_release);
    }
  }
  return NULL;
}

/*
 * The oracle's reduction with the sweeps of each pass on host threads.
 * nthreads > 0: min(nthreads, sweeps of the pass) threads, exactly.
 * nthreads < 0: at most -nthreads, and per pass at most 2n/(3b) and n/256
 * (at least one), the page's caps that keep every thread's blocks busy
 * (page "A two-stage reduction on an Apple M5 Pro", section 6).
 * nthreads == 0: as nthreads < 0 with every online core.
 * Other arguments as bb_oracle_reduce; max_passes < 0
 * runs every pass, else only the first max_passes (a bounded timing sample;
 * d, e, band_out then hold the partly reduced band).  threads_used (optional)
 * receives the thread count.  Returns 0, or 1 on a bad argument or a thread
 * that could not be started.
 */
int SUF(bb_oracle_mt_reduce)(const REAL *band_in, int64_t ld_in, int64_t n, int bw, int tw, REAL *d, REAL *e,
                             REAL *band_out, int nthreads, int max_passes, int *threads_used) {
  geom_t gm;
  if (!band_in || make_geom(n, bw, tw, &gm) || ld_in < bw + 1) return ORC_ERR_ARG;
  const int capped = nthreads <= 0;
  if (nthreads == 0) nthreads = bb_oracle_mt_default_threads();
  if (nthreads < 0) nthreads = -nthreads;
  REAL *a = SUF(load_band)(band_in, ld_in, bw, &gm);
  _Atomic int64_t *done = (_Atomic int64_t *)calloc((size_t)(n + 1), sizeof(_Atomic int64_t));
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  SUF(mt_job_t) *jobs = (SUF(mt_job_t) *)malloc(sizeof(SUF(mt_job_t)) * (size_t)nthreads);
  int rc = (a && done && tid && jobs) ? ORC_OK : ORC_ERR_ARG;
  int passes = 0, used = 0;
  for (int64_t b = bw; rc == ORC_OK && b > 1 && (max_passes < 0 || passes < max_passes);) {
    const int64_t t = (tw < b - 1) ? tw : b - 1;
    const int64_t bp = b - t;
    const int64_t ns = n - bp - 1 > 0 ? n - bp - 1 : 0;
    int64_t cap = nthreads;
    if (capped) {
      cap = min64(cap, min64(2 * n / (3 * b), n / 256));
      if (cap < 1) cap = 1;
    }
    const int P = (int)(ns < cap ? (ns > 0 ? ns : 1) : cap);
    for (int64_t R = 0; R < ns; ++R) atomic_store_explicit(&done[R], 0, memory_order_relaxed);
    int started = 0;
    for (int p = 0; p < P; ++p) {
      jobs[p].a = a;
      jobs[p].gm = &gm;
      jobs[p].b = b;
      jobs[p].t = t;
      jobs[p].ns = ns;
      jobs[p].lag = (bp >= 2) ? 2 : 3;
      jobs[p].nthreads = P;
      jobs[p].id = p;
      jobs[p].done = done;
      if (pthread_create(&tid[p], NULL, SUF(mt_worker), &jobs[p]) != 0) {
        rc = ORC_ERR_ARG;
        break;
      }
      ++started;
    }
    /* a thread that failed to start leaves its sweeps undone and its
     * successors waiting: only possible before any sweep has run, so give up */
    if (started < P) {
      fprintf(stderr, "bb_oracle_mt: could not start thread %d of %d\n", started, P);
      abort();
    }
    for (int p = 0; p < started; ++p) pthread_join(tid[p], NULL);
    if (P > used) used = P;
    b = bp;
    ++passes;
  }
  if (rc == ORC_OK) SUF(store_out)(a, &gm, d, e, band_out);
  free(a);
  free((void *)done);
  free(tid);
  free(jobs);
  if (threads_used) *threads_used = used;
  return rc;
}
