// HIP kernels (gfx950) of the band -> bidiagonal reduction.
//
// One cycle of a sweep (page "Accelerating Bidiagonalization of Banded
// Matrices through Memory-Aware Bulge-Chasing on GPUs", Algorithm 2
// passage): the t+1 entries of the row to annihilate are staged in LDS, every
// thread forms the Householder reflector from them, then each thread owns one
// row of the right-apply block (t+1 entries in VGPRs), applies the reflector
// and writes the row back; the same is repeated for the leftmost column of
// the bulge just created, one thread per column of the left-apply block.
//
// Arithmetic contract (so that results are reproducible to the bit by any
// implementation following it): reflector H = I - tau v v^T with
// v = (1, x_j / (alpha - beta)), beta = -sign(alpha) ||x|| (sign(+-0) = +1),
// tau = (beta - alpha) / beta; the tail sum of squares and every dot product
// are serial in increasing index with fused multiply-adds, nothing else is
// contracted (-ffp-contract=off), square root and division are correctly
// rounded.  A zero tail makes the reflector the identity; the annihilated
// entries are written as exact zeros either way.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_internal.hpp"

namespace bb {
namespace {

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float sqrt_(float a) { return __builtin_sqrtf(a); }
__device__ __forceinline__ double sqrt_(double a) { return __builtin_sqrt(a); }

template <typename T>
struct Refl {
  T beta, tau, inv;
  bool nz;  // false: identity (zero tail)
};

// Reflector of x[0..m-1] (x in LDS, read by every thread: broadcast).
template <typename T, int MAXM>
__device__ __forceinline__ Refl<T> house(const T *x, int m) {
  Refl<T> h;
  const T alpha = x[0];
  T s = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (j < m) s = fma_(x[j], x[j], s);
  if (s == T(0)) {
    h.nz = false;
    h.beta = alpha;
    h.tau = T(0);
    h.inv = T(0);
    return h;
  }
  const T nrm = sqrt_(fma_(alpha, alpha, s));
  h.beta = (alpha >= T(0)) ? -nrm : nrm;
  h.tau = (h.beta - alpha) / h.beta;
  h.inv = T(1) / (alpha - h.beta);
  h.nz = true;
  return h;
}

// Band view: element (i, j) at a[i*ld + (j - i + sub)].
template <typename T>
struct BandRef {
  T *a;
  int64_t ld;
  int32_t sub;
  int64_t n;
  __device__ __forceinline__ int64_t idx(int64_t i, int64_t j) const { return i * ld + (j - i + sub); }
};

// One cycle (R, k) of the pass (b, t), executed by the whole workgroup.
// xs, ys: LDS vectors of MAXM entries.  The caller guarantees the cycle
// exists (c <= n-2) and that no other workgroup touches its window.
template <typename T, int MAXM>
__device__ void block_cycle(const BandRef<T> A, int b, int t, int64_t R, int64_t k, T *xs, T *ys) {
  const int64_t n = A.n;
  const int64_t c = R + (b - t) + k * b;
  const int64_t ch = c + t < n - 1 ? c + t : n - 1;
  const int m = int(ch - c + 1);
  const int64_t r = (k == 0) ? R : c - b;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;

  // 1. row reflector from A(r, c..ch), staged in LDS
  if (tid < m) xs[tid] = A.a[A.idx(r, c + tid)];
  __syncthreads();
  const Refl<T> h = house<T, MAXM>(xs, m);

  // right apply: one row i = r+1..ch per thread, its m entries in VGPRs.
  // Column c of rows c..ch (the next reflector's input) goes to LDS only;
  // the column step writes it to memory.
  for (int64_t i = r + 1 + tid; i <= ch; i += nt) {
    T *p = A.a + A.idx(i, c);
    T v[MAXM];
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j < m) v[j] = p[j];
    if (h.nz) {
      T s = T(0);
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (j < m) s = fma_(v[j], xs[j], s);
      const T w = fma_(s, h.inv, v[0]);
      const T tw = h.tau * w;
      v[0] = v[0] - tw;
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (j < m) v[j] = fma_(-tw, xs[j] * h.inv, v[j]);
#pragma unroll
      for (int j = 1; j < MAXM; ++j)
        if (j < m) p[j] = v[j];
    }
    if (i >= c)
      ys[i - c] = v[0];
    else if (h.nz)
      p[0] = v[0];
  }
  if (tid == nt - 1) {
    if (h.nz) A.a[A.idx(r, c)] = h.beta;
    for (int j = 1; j < m; ++j) A.a[A.idx(r, c + j)] = T(0);
  }
  __syncthreads();

  // 2. column reflector from the updated A(c..ch, c) in LDS
  const Refl<T> g = house<T, MAXM>(ys, m);
  const int64_t jend = c + t + b < n - 1 ? c + t + b : n - 1;
  if (g.nz) {
    const int64_t st = A.ld - 1;  // (c+i, j) sits i*(ld-1) after (c, j)
    for (int64_t j = c + 1 + tid; j <= jend; j += nt) {
      T *p = A.a + A.idx(c, j);
      T v[MAXM];
#pragma unroll
      for (int i = 0; i < MAXM; ++i)
        if (i < m) v[i] = p[i * st];
      T s = T(0);
#pragma unroll
      for (int i = 1; i < MAXM; ++i)
        if (i < m) s = fma_(ys[i], v[i], s);
      const T w = fma_(s, g.inv, v[0]);
      const T tw = g.tau * w;
      v[0] = v[0] - tw;
#pragma unroll
      for (int i = 1; i < MAXM; ++i)
        if (i < m) v[i] = fma_(-tw, ys[i] * g.inv, v[i]);
#pragma unroll
      for (int i = 0; i < MAXM; ++i)
        if (i < m) p[i * st] = v[i];
    }
  }
  if (tid == nt - 1) {
    A.a[A.idx(c, c)] = g.nz ? g.beta : ys[0];
    for (int i = 1; i < m; ++i) A.a[A.idx(c + i, c)] = T(0);
  }
}

// One launch per step L of a pass: block q runs sweep R = Rlo + q, cycle
// k = L - s R (page: Algorithm 1, one kernel launch per cycle, kernel
// completion as the synchronisation).
template <typename T, int MAXM>
__global__ void __launch_bounds__(256) k_step(BandRef<T> A, int b, int t, int64_t L, int s, int64_t Rlo) {
  __shared__ T xs[MAXM];
  __shared__ T ys[MAXM];
  const int64_t R = Rlo + blockIdx.x;
  block_cycle<T, MAXM>(A, b, t, R, L - int64_t(s) * R, xs, ys);
}

// User band (row-offset layout) -> working band with zeroed bulge room.
template <typename T>
__global__ void k_pack(const T *__restrict__ band, int64_t ld_band, int64_t n, int bw, T *__restrict__ a,
                       int64_t ld, int sub) {
  const int64_t total = n * ld;
  for (int64_t q = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; q < total;
       q += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i = q / ld;
    const int64_t o = q - i * ld - sub;  // j - i
    T v = T(0);
    if (o >= 0 && o <= bw && i + o < n) v = band[i * ld_band + o];
    a[q] = v;
  }
}

template <typename T>
__global__ void k_extract(const T *__restrict__ a, int64_t ld, int sub, int64_t n, T *__restrict__ d,
                          T *__restrict__ e) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    d[i] = a[i * ld + sub];
    if (e != nullptr && i + 1 < n) e[i] = (ld > sub + 1) ? a[i * ld + sub + 1] : T(0);
  }
}

__global__ void k_fill_u32(uint32_t *p, int64_t count, uint32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

inline unsigned grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return unsigned(g);
}

template <typename T, int MAXM>
hipError_t step_t(void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo, int64_t nblk,
                  int nt, hipStream_t st) {
  BandRef<T> A{static_cast<T *>(wband), g.ld, g.sub, g.n};
  hipLaunchKernelGGL((k_step<T, MAXM>), dim3(unsigned(nblk)), dim3(nt), 0, st, A, b, t, L, s, Rlo);
  return hipGetLastError();
}

template <typename T>
hipError_t step_dispatch(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                         int64_t nblk, int nt, hipStream_t st) {
  switch (maxm) {
    case 9: return step_t<T, 9>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 17: return step_t<T, 17>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 33: return step_t<T, 33>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    case 65: return step_t<T, 65>(wband, g, b, t, L, s, Rlo, nblk, nt, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_pack(const void *band, int64_t ld_band, void *wband, const Geometry &g, hipStream_t st) {
  const int block = 256;
  const unsigned grid = grid_for(g.n * g.ld, block);
  if (g.dtype == 1)
    hipLaunchKernelGGL(k_pack<double>, dim3(grid), dim3(block), 0, st, static_cast<const double *>(band), ld_band,
                       g.n, g.bw, static_cast<double *>(wband), int64_t(g.ld), g.sub);
  else
    hipLaunchKernelGGL(k_pack<float>, dim3(grid), dim3(block), 0, st, static_cast<const float *>(band), ld_band,
                       g.n, g.bw, static_cast<float *>(wband), int64_t(g.ld), g.sub);
  return hipGetLastError();
}

hipError_t launch_extract(const void *wband, const Geometry &g, void *d, void *e, hipStream_t st) {
  const int block = 256;
  const unsigned grid = grid_for(g.n, block);
  if (g.dtype == 1)
    hipLaunchKernelGGL(k_extract<double>, dim3(grid), dim3(block), 0, st, static_cast<const double *>(wband),
                       int64_t(g.ld), g.sub, g.n, static_cast<double *>(d), static_cast<double *>(e));
  else
    hipLaunchKernelGGL(k_extract<float>, dim3(grid), dim3(block), 0, st, static_cast<const float *>(wband),
                       int64_t(g.ld), g.sub, g.n, static_cast<float *>(d), static_cast<float *>(e));
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t *p, int64_t count, uint32_t v, hipStream_t st) {
  const int block = 256;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(count, block)), dim3(block), 0, st, p, count, v);
  return hipGetLastError();
}

hipError_t launch_step(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                       int64_t nblk, int nt, hipStream_t st) {
  if (g.dtype == 1) return step_dispatch<double>(maxm, wband, g, b, t, L, s, Rlo, nblk, nt, st);
  return step_dispatch<float>(maxm, wband, g, b, t, L, s, Rlo, nblk, nt, st);
}

}  // namespace bb
