/*
 * bb.h -- C ABI of the MI355X (gfx950) band -> bidiagonal reduction library.
 *
 * The library reduces an upper-banded n x n matrix A of bandwidth BW
 * (A(i,j) != 0 only for 0 <= j-i <= BW) to upper bidiagonal form
 * B = Q^T A P by Householder bulge chasing with successive band reduction:
 * each pass removes t = min(TW, b-1) diagonals of the current bandwidth b,
 * down to b = 1.  A sweep per row annihilates one group of the row and one
 * group of the column it fills per cycle, and chases the bulge down the band;
 * consecutive sweeps run concurrently under the page's non-overlap rule.
 * Defined by the page "Accelerating Bidiagonalization of Banded Matrices
 * through Memory-Aware Bulge-Chasing on GPUs" (three-cycle-separation
 * passage; Algorithm 2 memory-strategy passage) and the page "A two-stage
 * reduction on an Apple M5 Pro", section 6 (sweep s may run its step once
 * sweep s-1 has finished the step two ahead).
 *
 * Conventions for every entry point:
 *   - All pointers named "device" are HIP device pointers; "host" pointers
 *     are ordinary host memory.  The caller owns every buffer and the stream;
 *     the library allocates no device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; results are ready once the
 *     stream has been synchronised.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns an error and enqueues nothing.  No C++ exception
 *     crosses this interface.
 *   - dtype is BB_F32, BB_F64 or BB_F16 (see bb_dtype) and is both the
 *     storage and the arithmetic precision of the reduction.
 *   - Values are not checked for NaN/Inf; non-finite input propagates.
 */
#ifndef BB_H_
#define BB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage and arithmetic precision.  BB_F16 (IEEE binary16) is the
 * reduced-precision variant of the band -> bidiagonal reduction (page
 * "Accelerating Bidiagonalization of Banded Matrices through Memory-Aware
 * Bulge-Chasing on GPUs", the accuracy study run in FP64, FP32 and FP16):
 * bb_reduce and its staged entry points only, on every scheduler but STEP;
 * each operation rounded once to fp16 (fma fused, sqrt and division
 * correctly rounded).  The symmetric reduction and bb_svals take BB_F32 and
 * BB_F64. */
typedef enum { BB_F32 = 0, BB_F64 = 1, BB_F16 = 2 } bb_dtype;

typedef enum {
  BB_OK = 0,
  BB_ERR_ARG = 1,          /* invalid size, pointer or dtype */
  BB_ERR_WORKSPACE = 2,    /* work_bytes below bb_workspace_bytes() */
  BB_ERR_HIP = 3,          /* a HIP call or kernel launch failed */
  BB_ERR_UNSUPPORTED = 4,  /* valid but not implemented: tile width > 64, a
                              pass whose (b+t+1) x (t+1) blocks exceed LDS,
                              or a band of 2 GiB or more */
  BB_ERR_TIMEOUT = 5       /* a device-side bounded wait expired */
} bb_status;

/* Schedulers of the sweeps (page: Algorithm 1 launches one kernel per cycle
 * with kernel completion as the synchronisation). */
typedef enum {
  BB_SCHED_DEFAULT = 0,   /* the fastest scheduler for the shape */
  BB_SCHED_STEP = 1,      /* one launch per step: step L runs every (R, k=L-s*R) */
  BB_SCHED_PERSISTENT = 2, /* resident workgroups; per-sweep progress counters */
  BB_SCHED_GROUP = 3,      /* resident workgroups each running a group of
                              consecutive sweeps on a ring of band rows in LDS
                              (tile widths up to 16; 31 and 32 in fp32 and 31
                              in fp64 on rings of row windows, the entries a
                              pass touches); passes whose ring does not fit
                              run PERSISTENT; one launch per pass (DEFAULT
                              also lets consecutive group passes share a
                              launch, windowed ones excepted) */
  BB_SCHED_BARRIER = 4     /* one launch per pass of resident workgroups (one
                              per CU, at most max_blocks) running STEP's steps
                              with a device-wide barrier between steps; fp32
                              and fp64 only, general band only */
} bb_scheduler;

/* Optional tuning; pass NULL for the gfx950 defaults.  Zero fields take the
 * default. */
typedef struct {
  int32_t scheduler;         /* bb_scheduler */
  int32_t stagger;           /* cycles between consecutive sweeps: 0 = the
                                smallest safe value (2 when the pass's target
                                bandwidth b' > 1, else 3); 3 = always three */
  int32_t max_blocks;        /* persistent, group: resident workgroups (0 = device fill) */
  int32_t threads_per_block; /* 64..256, multiple of 64 (0 = default) */
  int64_t spin_limit;        /* persistent, group: bound of every device-side
                                wait, in microseconds (0 = 2 s, at most 20 s):
                                a wait that outlasts it, or any wait running
                                when another has expired, stops; every
                                workgroup of the launch then drains, and
                                bb_device_status reports BB_ERR_TIMEOUT */
  int32_t group_sweeps;      /* group: sweeps per workgroup, 1..6 (0 = the most that fit) */
  int32_t reserved;          /* must be 0 */
} bb_tuning;

/* Host-side plan of a reduction (no device work). */
typedef struct {
  int32_t passes;     /* number of band-reduction passes */
  int32_t ld;         /* stored diagonals per row of the working band */
  int32_t sub;        /* sub-diagonals stored (fill below the diagonal) */
  int32_t reserved;
  int64_t sweeps;     /* sweeps over all passes */
  int64_t cycles;     /* cycles over all passes */
  int64_t steps;      /* dependent steps at three-cycle stagger, all passes */
  double alg_bytes;   /* algorithmic bytes: per cycle, read + write of the
                         union of its row block and column block */
  double flops;       /* floating-point operations of all reflectors/applies */
} bb_plan_info;

/* Plan for (n, bw, tw, dtype): the pass list (page "Accelerating
 * Bidiagonalization of Banded Matrices through Memory-Aware Bulge-Chasing on
 * GPUs", bandwidth-tiling passage: each pass takes TW diagonals off the
 * current bandwidth), the sweeps and cycles of each pass (same page, the
 * passage on the cycle's window moving BW down the band per cycle), and the
 * algorithmic bytes by which that page's profiling section rates the kernel.
 * out: host pointer.  Errors: BB_ERR_ARG. */
bb_status bb_plan(int64_t n, int32_t bw, int32_t tw, int32_t dtype, bb_plan_info *out);

/* Bytes of device workspace bb_reduce needs: the working band, whose rows
 * hold the bw + 2 min(tw, bw-1) + 1 diagonals a pass's bulges can reach
 * (page "Accelerating Bidiagonalization of Banded Matrices through
 * Memory-Aware Bulge-Chasing on GPUs": a cycle's window spans 1 + BW + TW
 * entries in each direction), plus the schedulers' counters.
 * bytes: host pointer.  Errors: BB_ERR_ARG, BB_ERR_UNSUPPORTED. */
bb_status bb_workspace_bytes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, size_t *bytes);

/*
 * Reduces the band to bidiagonal form: every pass, sweep and cycle of the
 * page "Accelerating Bidiagonalization of Banded Matrices through
 * Memory-Aware Bulge-Chasing on GPUs" (Algorithm 1: the sweeps' schedule;
 * Algorithm 2: one cycle's row and column reflectors and their applies), in
 * the order of the sequential chase of the page "A two-stage reduction on an
 * Apple M5 Pro", section 6, whose results it reproduces bit for bit.
 *   band     device, read only: row i holds A(i, i+o) at band[i*ld_band + o],
 *            o = 0..bw; entries with i+o >= n are ignored.
 *   ld_band  >= bw + 1 (elements).
 *   n >= 1, bw >= 0, tw >= 1 (clamped per pass to b-1).
 *   d        device, n entries: d[i] = B(i,i).
 *   e        device, n-1 entries: e[i] = B(i,i+1) (may be NULL when n == 1).
 *            Signs are those the reflectors produce (not normalised).
 *   work     device workspace of work_bytes >= bb_workspace_bytes(); its
 *            contents on entry do not matter; it holds the working band and
 *            the scheduler's counters afterwards.  Distinct concurrent calls
 *            need distinct workspaces.
 *   tuning   host pointer or NULL.
 *   stream   hipStream_t as void*.
 * bw <= 1 copies the band out.  Errors: BB_ERR_ARG, BB_ERR_WORKSPACE,
 * BB_ERR_UNSUPPORTED, BB_ERR_HIP (launch failure).
 */
bb_status bb_reduce(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype,
                    void *d, void *e, void *work, size_t work_bytes, const bb_tuning *tuning, void *stream);

/* Largest workspace bb_reduce_noalloc can use: 16 MiB per GPU. */
#define BB_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * bb_reduce for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same reduction with the same results, bit for bit, but with no `work`
 * argument.  Its workspace is a fixed array of BB_NOALLOC_SCRATCH_BYTES in
 * the library's code object, one per GPU, held until the process ends; the
 * call allocates nothing (no hipMalloc, no allocating library routine).
 *   band, ld_band, n, bw, tw, dtype, d, e, tuning, stream: as for bb_reduce,
 *            on the device current at the call.
 *   status   device pointer to one uint32_t, or NULL: receives the launch's
 *            status word when the reduction is done (0 = completed, nonzero =
 *            a bounded wait expired, as bb_device_status reports it).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the call resets what must start at zero): calls that overlap on
 * one GPU (concurrent streams, or host threads) race and must be serialised
 * by the caller.  Errors: as bb_reduce, and BB_ERR_WORKSPACE when the shape
 * needs more than BB_NOALLOC_SCRATCH_BYTES (bb_workspace_bytes); n = 16384,
 * bw = 64, tw = 16 fp32 needs 8.3 MiB.
 */
bb_status bb_reduce_noalloc(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype,
                            void *d, void *e, void *status, const bb_tuning *tuning, void *stream);

/*
 * The three stages bb_reduce runs, for callers that time or interleave them:
 * bb_pack, then bb_run_passes over passes 0 .. passes-1 (in one call, or
 * split into consecutive ranges, or bb_run_pass for each pass in order), then
 * bb_extract, all on one stream, equal bb_reduce with the same arguments
 * (bit for bit, however the passes are split).
 *
 * bb_pack: resets the counters in `work` and copies the caller's band (same
 *   layout and requirements as bb_reduce's `band`, `ld_band`) into the
 *   working band with zeroed room for the bulge.
 * bb_run_pass: runs pass `pass` (0-based; the pass list takes the bandwidth
 *   b -> b - min(tw, b-1) until it reaches 1, page "Accelerating
 *   Bidiagonalization of Banded Matrices through Memory-Aware Bulge-Chasing
 *   on GPUs", tile-width passage) on the working band in `work`; every
 *   earlier pass must have run on it.  tuning as for bb_reduce.
 * bb_run_passes: runs passes first .. first+count-1 (count >= 0) in order,
 *   as bb_run_pass would one by one.  Under BB_SCHED_DEFAULT, consecutive
 *   passes that run on the LDS group kernel with register tiles of one
 *   family (8/9 or 16/17 entries) share one launch, at most 4 passes each:
 *   the first sweep group of a pass starts on rows the previous pass is done
 *   with while that pass still runs (each row's owner in the previous pass
 *   publishes when it is done with the row).  bb_run_pass never shares a
 *   launch.
 * bb_extract: writes d and e (as for bb_reduce) from the working band.
 * Errors: BB_ERR_ARG (also for pass out of range), BB_ERR_WORKSPACE,
 * BB_ERR_UNSUPPORTED, BB_ERR_HIP.
 */
bb_status bb_pack(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *work,
                  size_t work_bytes, void *stream);
bb_status bb_run_pass(int64_t n, int32_t bw, int32_t tw, int32_t dtype, int32_t pass, void *work, size_t work_bytes,
                      const bb_tuning *tuning, void *stream);
bb_status bb_run_passes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, int32_t first, int32_t count, void *work,
                        size_t work_bytes, const bb_tuning *tuning, void *stream);
bb_status bb_extract(const void *work, size_t work_bytes, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *d,
                     void *e, void *stream);

/* The cycle-kernel launches bb_run_passes makes for all passes with this
 * tuning (host only, no device work): *launches = their number; when
 * capacity > 0 (it must then be >= the number of passes), launch_of_pass[p] =
 * the index of the launch that runs pass p, -1 for a pass without sweeps.
 * launch_of_pass, launches: host pointers.  Errors: BB_ERR_ARG,
 * BB_ERR_UNSUPPORTED (also fp16 with BB_SCHED_STEP, as bb_run_passes). */
bb_status bb_launch_plan(int64_t n, int32_t bw, int32_t tw, int32_t dtype, const bb_tuning *tuning,
                         int32_t *launch_of_pass, int32_t capacity, int32_t *launches);

/* Copies the working band left in `work` by the last bb_reduce with the same
 * (n, bw, tw, dtype) -- the whole matrix state after the passes, fill and
 * annihilated entries included (page "Accelerating Bidiagonalization of
 * Banded Matrices through Memory-Aware Bulge-Chasing on GPUs", Algorithm 2
 * passage: annihilated entries are written back as zeros) -- to dst (device, n * ld elements of dtype; element (i,j)
 * at dst[i*ld + j-i+sub] with ld, sub from bb_plan).  Errors: BB_ERR_ARG,
 * BB_ERR_HIP. */
bb_status bb_export_band(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *dst,
                         void *stream);

/* Synchronises `stream` and reports the device-side status word of the
 * last bb_reduce on `work` (BB_OK or BB_ERR_TIMEOUT): whether every bounded
 * wait of the sweep dependency rule (page "A two-stage reduction on an Apple
 * M5 Pro", section 6: a sweep waits until the previous sweep has finished
 * the step two ahead) ended before its bound.  Errors: BB_ERR_ARG,
 * BB_ERR_HIP. */
bb_status bb_device_status(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *stream);

/* ---- Symmetric band -> tridiagonal ----
 *
 * Defined by the page "A two-stage reduction on an Apple M5 Pro", section 6
 * (the band chase with the symmetric-band kernels): a symmetric n x n matrix
 * of bandwidth BW (A(i,j) = 0 for |i-j| > BW) is reduced to tridiagonal form
 * T = Q^T A Q by the same passes (b -> b - t, t = min(TW, b-1); TW >= BW-1 is
 * one pass), sweeps and cycles as the general band, with one reflector per
 * cycle applied from both sides: from the row segment A(p, c..ch) to rows
 * p+1..c-1 and the symmetric block c..ch and columns ch+1..ch+b.
 *   band   device, row i (stride ld_band >= bw+1 elements) holds
 *          A(i, i..i+bw) = A(i..i+bw, i); entries past n are ignored.
 *   d, e   device outputs: d[i] = T(i,i) (n), e[i] = T(i,i+1) (n-1; may be
 *          NULL when n == 1).  e is determined up to sign.
 *   work   device workspace, 256-byte aligned, of bb_sym_workspace_bytes();
 *          the working band (row i at i*stride, element (i,j) at offset j-i,
 *          W+1 = bw + min(tw,bw-1) + 1 entries in use) and counters.
 *   tuning NULL or as for bb_reduce: DEFAULT and GROUP run sweep groups
 *          resident in LDS where the pass fits (tile widths up to 16, or 32
 *          in fp32), else PERSISTENT; STEP is not available.
 * Same arithmetic contract as bb_reduce; the reduction of the symmetric
 * block uses LAPACK's rank-2 form y = tau B v, alpha = -(tau/2) y.v,
 * z = y + alpha v, B -= v z^T + z v^T, every sum serial with fma.
 * The sweeps run by half-cycles (the pivot row and the row segments; the
 * block and the column segments) with the lag of the general band.
 * Errors: BB_ERR_ARG, BB_ERR_UNSUPPORTED (tile width > 64, band of 2 GiB or
 * more, the STEP scheduler, BB_F16), BB_ERR_WORKSPACE,
 * BB_ERR_HIP.  bb_sym_device_status reports BB_ERR_TIMEOUT after a bounded
 * wait expired. */
bb_status bb_sym_workspace_bytes(int64_t n, int32_t bw, int32_t tw, int32_t dtype, size_t *bytes);
bb_status bb_sym_reduce(const void *band, int64_t ld_band, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *d,
                        void *e, void *work, size_t work_bytes, const bb_tuning *tuning, void *stream);

/* Copies the symmetric working band left in `work` to dst (device, n rows
 * of W+1 elements, row i = A(i, i..i+W)).  Errors: BB_ERR_ARG, BB_ERR_HIP. */
bb_status bb_sym_export_band(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *dst,
                             void *stream);

/* Synchronises `stream`; BB_OK or BB_ERR_TIMEOUT for the last bb_sym_reduce
 * on `work`.  Errors: BB_ERR_ARG, BB_ERR_HIP. */
bb_status bb_sym_device_status(const void *work, int64_t n, int32_t bw, int32_t tw, int32_t dtype, void *stream);

/* ---- Singular values of the bidiagonal (the step after the reduction) ----
 *
 * Defined by the page "A two-stage reduction on an Apple M5 Pro", section 7:
 * the singular values of the upper bidiagonal B (diagonal d, superdiagonal e)
 * are the non-negative eigenvalues of the 2n x 2n Golub-Kahan tridiagonal
 * (zero diagonal, off-diagonal d_0, e_0, d_1, ..., d_{n-1}); each is found by
 * bisection from its Gershgorin interval with a fixed number of halvings
 * (26 in fp32, 55 in fp64), each a Sturm count with LAPACK's pivmin guard.
 * The result is absolutely accurate: within a few ulps of max sigma.  It is
 * the same to the bit for every `levels`, and deterministic.
 */

/* Device workspace bytes for bb_svals on an order-n bidiagonal.
 * Errors: BB_ERR_ARG (n < 0, n > 2^29, bad dtype, bytes NULL). */
bb_status bb_svals_workspace_bytes(int64_t n, int32_t dtype, size_t *bytes);

/* Singular values i0 .. i1-1 of B in descending order (sigma_0 is the
 * largest), 0 <= i0 <= i1 <= n, written to sigma[0 .. i1-i0-1].
 *   d      device, n elements of dtype; e device, n-1 elements (unused, may
 *          be NULL, when n == 1).  Signs of d and e do not matter.
 *   tree_levels  the first K halvings, shared by every value, are counted
 *          once for all 2^K - 1 nodes of the top of the bisection tree
 *          (1 .. 16); -1 = none, 0 = chosen for the size.
 *   levels then D halvings per round, a group of 2^D lanes per value
 *          (1 .. 6); 0 = chosen for the size.
 *          Only the speed depends on K and D: the values are the same bits.
 *   work   device workspace of work_bytes >= bb_svals_workspace_bytes(),
 *          256-byte aligned, owned by the caller, overwritten.
 * Enqueues up to three kernels on `stream`; nothing when n == 0 or i0 == i1.
 * Errors: BB_ERR_ARG (sizes, range, NULL or misaligned pointers, K, D),
 * BB_ERR_WORKSPACE, BB_ERR_HIP. */
bb_status bb_svals(const void *d, const void *e, int64_t n, int32_t dtype, int64_t i0, int64_t i1,
                   int32_t tree_levels, int32_t levels, void *sigma, void *work, size_t work_bytes, void *stream);

/* The (tree_levels, levels) bb_svals picks for `values` singular values on
 * the current device.  Errors: BB_ERR_ARG. */
bb_status bb_svals_split(int64_t values, int32_t dtype, int32_t *tree_levels, int32_t *levels);

/* Static description of a status code. */
const char *bb_status_str(int32_t status);

/* ---- Measurement probes (not part of the reduction) ----------------------
 * Bandwidth ceilings for the memory level that holds a working band, for
 * the cycle kernels' roofline (page "Accelerating Bidiagonalization of Banded
 * Matrices through Memory-Aware Bulge-Chasing on GPUs", profiling section:
 * runtime tracks the throughput of the cache levels, and a matrix
 * transpose-add is the reference point for row- and column-wise access).
 * Both enqueue one kernel on `stream` and return at once; the caller times
 * them and owns every buffer.  The kernel repeats the operation `reps` >= 1
 * times, handing each element to another workgroup (so another XCD) on each
 * repetition; the result does not depend on `reps`.
 *
 * z[i] = x[i] + y[i], i < n, fp32, 16-byte accesses with the cycle kernels'
 * agent-coherent cache policy: 12 n bytes move per repetition.  x, y, z:
 * device, 16-byte aligned, z distinct from x and y; n a multiple of 4,
 * 4 n bytes < 2 GiB.  Errors: BB_ERR_ARG, BB_ERR_HIP. */
bb_status bb_probe_stream(const void *x, const void *y, void *z, int64_t n, int32_t reps, void *stream);

/* B = A + A^T for an m x m row-major fp32 matrix, through LDS tiles (both
 * reads coalesced): 12 m^2 bytes move per repetition.  a, b: device,
 * distinct; m^2 <= 2^30.  Errors: BB_ERR_ARG, BB_ERR_HIP. */
bb_status bb_probe_transpose_add(const void *a, void *b, int32_t m, int32_t reps, void *stream);

/* Shader clocks of `reps` dependent reflector norms (the sum of squares of
 * m - 1 fp32 entries) in one wave: mode 0 sums serially with FMAs in every
 * lane (the reduction's own order, page "Accelerating Bidiagonalization of
 * Banded Matrices through Memory-Aware Bulge-Chasing on GPUs", Algorithm 2
 * memory-strategy passage: the TW+1 staged entries form the reflector),
 * mode 1 by a DPP cross-lane reduction, one entry per lane.  m: 17 or 33;
 * x: device, 64 floats; out: device, 64 floats (scratch); clocks: device,
 * one uint64 (written).  Errors: BB_ERR_ARG, BB_ERR_HIP. */
bb_status bb_probe_norm_clocks(int32_t m, int32_t mode, int32_t reps, const void *x, void *out, void *clocks,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BB_H_ */
