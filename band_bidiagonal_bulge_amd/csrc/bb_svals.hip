// Singular values of an upper bidiagonal matrix by bisection, the step after
// the band -> bidiagonal reduction (page "A two-stage reduction on an Apple
// M5 Pro", section 7).
//
// The singular values of B (diagonal d, superdiagonal e) are the non-negative
// eigenvalues of the 2n x 2n Golub-Kahan tridiagonal T: zero diagonal,
// off-diagonal b_1..b_{2n-1} = d_0, e_0, d_1, ..., d_{n-1}.  Each eigenvalue
// is bisected on its own from T's Gershgorin interval with a fixed number of
// halvings; a halving keeps the half that holds the eigenvalue by a Sturm
// count (eigenvalues of T <= x, the number of non-positive pivots of
// T - xI = LDL^T) with LAPACK's guard against tiny pivots.
//
// The constants, the count and the interval follow one reading of the page,
// fixed so that the result is reproducible to the bit:
//   count(x):  q_1 = -x, q_j = -(bb_{j-1} / q_{j-1}) - x, bb_j = b_j * b_j;
//              |q_j| < pivmin -> q_j = -pivmin; count the q_j <= 0
//   pivmin   = smallest normal * max(1, max bb)
//   interval = [-(r + delta), r + delta], r = max_i |b_{i-1}| + |b_i|,
//              delta = ((r * 2n) * eps) + 2 pivmin
//   p + 2 halvings (26 fp32, 55 fp64): mid = 0.5 (lo + hi), keep [lo, mid]
//              when count(mid) >= j (ascending 1-based index j = 2n - i)
//   sigma_i  = 0.5 (lo + hi) of the last interval, +0 if not positive.
// Every operation is rounded on its own (built with -ffp-contract=off;
// division is the correctly rounded one).
//
// gfx950 mapping.  One bisection is a chain of p + 2 counts, each a serial
// recurrence over 2n pivots: latency, not bandwidth, is the problem, and one
// lane per eigenvalue leaves most SIMDs idle at the sizes of interest.  So a
// group of L lanes bisects one eigenvalue, D levels per round: lane h-1
// evaluates the count at node h (1 <= h < 2^D) of the depth-D subtree of the
// bisection below the current interval, the wave ballots "count >= j", and
// every lane walks the subtree from the root with the ballot's bits.  The
// walk recomputes each midpoint from the same operands the serial bisection
// would use, so D levels per round give exactly the serial result with
// ceil((p+2)/D) counts in the chain instead of p+2.  The host picks D from
// the number of values and the SIMD count.  The squared off-diagonal is
// prepared once (k_gk_prep) and read by every wave in 64-entry chunks, one
// entry per lane, broadcast to the recurrence with v_readlane; the next chunk
// is in flight while the current one is consumed.

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstdint>

#include "bb_internal.hpp"

namespace bb {
namespace {

template <typename T>
struct Lim;
template <>
struct Lim<float> {
  static constexpr float tiny = FLT_MIN;
  static constexpr float eps = FLT_EPSILON;
  static constexpr int halvings = FLT_MANT_DIG + 2;
};
template <>
struct Lim<double> {
  static constexpr double tiny = DBL_MIN;
  static constexpr double eps = DBL_EPSILON;
  static constexpr int halvings = DBL_MANT_DIG + 2;
};

// Off-diagonal entry j (1-based) of the Golub-Kahan tridiagonal.
template <typename T>
__device__ __forceinline__ T gk_b(const T *__restrict__ d, const T *__restrict__ e, int64_t j) {
  return (j & 1) ? d[(j - 1) >> 1] : e[(j >> 1) - 1];
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  for (int o = 32; o > 0; o >>= 1) {
    const T w = __shfl_xor(v, o, 64);
    v = (w > v) ? w : v;
  }
  return v;
}

// One workgroup of kPrepThreads: bb = b*b (zero-padded to the chunked length)
// and the header {lo, hi, pivmin}.  Maxima are exact, so their order is free.
template <typename T>
__global__ __launch_bounds__(kPrepThreads) void k_gk_prep(const T *__restrict__ d, const T *__restrict__ e,
                                                          int64_t n, int64_t padded, T *__restrict__ hdr,
                                                          T *__restrict__ bb) {
  __shared__ T red_bb[kPrepThreads / 64], red_r[kPrepThreads / 64];
  const int64_t m = 2 * n - 1;
  T mbb = 0, mr = 0;
  for (int64_t j = threadIdx.x + 1; j <= padded; j += kPrepThreads) {
    T v = 0;
    if (j <= m) {
      const T b = gk_b(d, e, j);
      v = b * b;
      mbb = (v > mbb) ? v : mbb;
    }
    bb[j - 1] = v;
  }
  for (int64_t i = threadIdx.x + 1; i <= 2 * n; i += kPrepThreads) {
    const T left = i > 1 ? fabs(gk_b(d, e, i - 1)) : T(0);
    const T right = i < 2 * n ? fabs(gk_b(d, e, i)) : T(0);
    const T s = left + right;
    mr = (s > mr) ? s : mr;
  }
  mbb = wave_max(mbb);
  mr = wave_max(mr);
  if ((threadIdx.x & 63) == 0) {
    red_bb[threadIdx.x >> 6] = mbb;
    red_r[threadIdx.x >> 6] = mr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kPrepThreads / 64; ++w) {
      mbb = (red_bb[w] > mbb) ? red_bb[w] : mbb;
      mr = (red_r[w] > mr) ? red_r[w] : mr;
    }
    const T pm = Lim<T>::tiny * (mbb > T(1) ? mbb : T(1));
    const T delta = ((mr * T(2 * n)) * Lim<T>::eps) + T(2) * pm;
    hdr[0] = -(mr + delta);
    hdr[1] = mr + delta;
    hdr[2] = pm;
  }
}

__device__ __forceinline__ float lane_value(float v, int s) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
}
__device__ __forceinline__ double lane_value(double v, int s) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(u), s);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(u >> 32), s);
  return __longlong_as_double((long long)((uint64_t(hi) << 32) | lo));
}

template <typename T>
__device__ __forceinline__ void pivot(T &q, int &c, T bbv, T x, T pm) {
  q = -(bbv / q) - x;
  q = (fabs(q) < pm) ? -pm : q;
  c += (q <= T(0)) ? 1 : 0;
}

// Number of eigenvalues of T that are <= x.  bb holds nb = 2n-1 entries,
// zero-padded to a multiple of 64 plus one spare chunk; lane = lane in wave.
template <typename T>
__device__ __forceinline__ int sturm_count(const T *__restrict__ bb, int nb, T x, T pm, int lane) {
  T q = -x;
  q = (fabs(q) < pm) ? -pm : q;
  int c = (q <= T(0)) ? 1 : 0;
  T cur = bb[lane];
  int base = 0;
  for (; base + 64 <= nb; base += 64) {
    const T nxt = bb[base + 64 + lane];
#pragma unroll
    for (int s = 0; s < 64; ++s) pivot(q, c, lane_value(cur, s), x, pm);
    cur = nxt;
  }
  for (int s = 0; s < nb - base; ++s) pivot(q, c, lane_value(cur, s), x, pm);
  return c;
}

// Value of node h (heap order: root 1, children 2h and 2h+1) of the
// bisection tree below [lo, hi]: the midpoints on its path, each from the
// same operands the serial bisection uses.
template <typename T>
__device__ __forceinline__ T node_value(T lo, T hi, int h) {
  for (int k = 30 - __builtin_clz(h); k >= 0; --k) {
    const T mid = T(0.5) * (lo + hi);
    if ((h >> k) & 1)
      lo = mid;
    else
      hi = mid;
  }
  return T(0.5) * (lo + hi);
}

// Counts at every node of the top K levels of the bisection tree below the
// Gershgorin interval: the levels every value's bisection shares.  One lane
// per node h = 1 .. 2^K - 1; every lane runs the count (the chunk broadcast
// reads all lanes' registers), only real nodes store.
template <typename T>
__global__ __launch_bounds__(kBisectThreads) void k_tree(const T *__restrict__ hdr, const T *__restrict__ bb,
                                                          int32_t n, int32_t K, int32_t *__restrict__ tree) {
  const int lane = threadIdx.x & 63;
  const int h = int(blockIdx.x) * kBisectThreads + int(threadIdx.x) + 1;
  const bool real = h < (1 << K);
  const T x = node_value(hdr[0], hdr[1], real ? h : 1);
  const int c = sturm_count(bb, 2 * n - 1, x, hdr[2], lane);
  if (real) tree[h] = c;
}

// Bisection of values i0 .. i1-1: first the K tree levels from the stored
// counts, then D levels per round by groups of L lanes (see the top).
template <typename T, int D>
__global__ __launch_bounds__(kBisectThreads) void k_bisect(const T *__restrict__ hdr, const T *__restrict__ bb,
                                                            const int32_t *__restrict__ tree, int32_t K,
                                                            int32_t n, int64_t i0, int64_t i1,
                                                            T *__restrict__ sigma) {
  constexpr int L = (D == 1) ? 1 : (1 << D);
  constexpr int F = Lim<T>::halvings;
  const int lane = threadIdx.x & 63;
  const int sub = threadIdx.x % L;  // this lane evaluates node sub + 1
  const int gbase = lane - sub;     // first lane of the group in the wave
  const int64_t i = i0 + (int64_t(blockIdx.x) * kBisectThreads + threadIdx.x) / L;
  const bool live = i < i1;
  const int32_t j = 2 * n - int32_t(live ? i : i0);
  const int nb = 2 * n - 1;
  const T pm = hdr[2];
  T lo = hdr[0], hi = hdr[1];
  for (int k = 0, node = 1; k < K; ++k) {
    const T mid = T(0.5) * (lo + hi);
    if (tree[node] >= j) {
      hi = mid;
      node = 2 * node;
    } else {
      lo = mid;
      node = 2 * node + 1;
    }
  }
  for (int done = K; done < F;) {
    const int lev = (F - done < D) ? F - done : D;
    const T x = node_value(lo, hi, sub + 1);
    const uint64_t below = __ballot(sturm_count(bb, nb, x, pm, lane) >= j);
    int node = 1;
    for (int k = 0; k < lev; ++k) {
      const T mid = T(0.5) * (lo + hi);
      if ((below >> (gbase + node - 1)) & 1ull) {
        hi = mid;
        node = 2 * node;
      } else {
        lo = mid;
        node = 2 * node + 1;
      }
    }
    done += lev;
  }
  if (live && sub == 0) {
    const T s = T(0.5) * (lo + hi);
    sigma[i - i0] = (s > T(0)) ? s : T(0);
  }
}

template <typename T>
const T *bb_of(const void *work) {
  return reinterpret_cast<const T *>(static_cast<const char *>(work) + kSvalsHeaderBytes + kSvalsTreeBytes);
}
const int32_t *tree_of(const void *work) {
  return reinterpret_cast<const int32_t *>(static_cast<const char *>(work) + kSvalsHeaderBytes);
}

template <typename T, int D>
hipError_t launch_bisect_t(const void *work, int64_t n, int K, int64_t i0, int64_t i1, void *sigma,
                           hipStream_t st) {
  constexpr int L = (D == 1) ? 1 : (1 << D);
  const int64_t threads = (i1 - i0) * L;
  const int64_t blocks = (threads + kBisectThreads - 1) / kBisectThreads;
  hipLaunchKernelGGL((k_bisect<T, D>), dim3(unsigned(blocks)), dim3(kBisectThreads), 0, st,
                     static_cast<const T *>(work), bb_of<T>(work), tree_of(work), int32_t(K), int32_t(n), i0, i1,
                     static_cast<T *>(sigma));
  return hipGetLastError();
}

template <typename T>
hipError_t launch_svals_t(int K, int D, void *work, int64_t n, int64_t i0, int64_t i1, void *sigma,
                          hipStream_t st) {
  if (K > 0) {
    const int64_t blocks = ((int64_t(1) << K) - 1 + kBisectThreads - 1) / kBisectThreads;
    hipLaunchKernelGGL(k_tree<T>, dim3(unsigned(blocks)), dim3(kBisectThreads), 0, st,
                       static_cast<const T *>(work), bb_of<T>(work), int32_t(n), int32_t(K),
                       reinterpret_cast<int32_t *>(static_cast<char *>(work) + kSvalsHeaderBytes));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  switch (D) {
    case 1: return launch_bisect_t<T, 1>(work, n, K, i0, i1, sigma, st);
    case 2: return launch_bisect_t<T, 2>(work, n, K, i0, i1, sigma, st);
    case 3: return launch_bisect_t<T, 3>(work, n, K, i0, i1, sigma, st);
    case 4: return launch_bisect_t<T, 4>(work, n, K, i0, i1, sigma, st);
    case 5: return launch_bisect_t<T, 5>(work, n, K, i0, i1, sigma, st);
    case 6: return launch_bisect_t<T, 6>(work, n, K, i0, i1, sigma, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t svals_padded_entries(int64_t n) { return ((2 * n - 1 + 63) / 64) * 64 + 64; }

int bisect_halvings(int dtype) { return dtype == 0 ? Lim<float>::halvings : Lim<double>::halvings; }

hipError_t launch_gk_prep(int dtype, const void *d, const void *e, int64_t n, void *work, hipStream_t st) {
  const int64_t padded = svals_padded_entries(n);
  char *w = static_cast<char *>(work);
  char *bbp = w + kSvalsHeaderBytes + kSvalsTreeBytes;
  if (dtype == 0)
    hipLaunchKernelGGL(k_gk_prep<float>, dim3(1), dim3(kPrepThreads), 0, st, static_cast<const float *>(d),
                       static_cast<const float *>(e), n, padded, reinterpret_cast<float *>(w),
                       reinterpret_cast<float *>(bbp));
  else
    hipLaunchKernelGGL(k_gk_prep<double>, dim3(1), dim3(kPrepThreads), 0, st, static_cast<const double *>(d),
                       static_cast<const double *>(e), n, padded, reinterpret_cast<double *>(w),
                       reinterpret_cast<double *>(bbp));
  return hipGetLastError();
}

hipError_t launch_svals(int dtype, int tree_levels, int levels, void *work, int64_t n, int64_t i0, int64_t i1,
                        void *sigma, hipStream_t st) {
  return dtype == 0 ? launch_svals_t<float>(tree_levels, levels, work, n, i0, i1, sigma, st)
                    : launch_svals_t<double>(tree_levels, levels, work, n, i0, i1, sigma, st);
}

}  // namespace bb
