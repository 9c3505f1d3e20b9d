// Symmetric band -> tridiagonal reduction by Householder bulge chasing
// (page "A two-stage reduction on an Apple M5 Pro", section 6: the band chase
// with the symmetric-band kernels; one reflector per step, a sweep clearing a
// row and chasing its bulge down the band a block of b at a time).
//
// The upper triangle of the band is stored (element (i, j), 0 <= j-i <= W, at
// row i, offset j-i).  Passes take the bandwidth b to b' = b - t.  Cycle k of
// sweep R, with c = R + b' + k b, ch = min(c+t, n-1), S = c..ch and pivot row
// p = R (k = 0) or c - b:
//   - H from the row segment A(p, S): A(p, c) = beta, A(p, c+1..ch) = 0;
//   - rows p+1..c-1 at columns S from the right (a row segment each);
//   - columns ch+1..min(ch+b, n-1) at rows S from the left (a column segment
//     each);
//   - the symmetric block S x S from both sides: y = tau B v,
//     alpha = -(tau/2) y.v, z = y + alpha v, B -= v z^T + z v^T.
// Arithmetic (reproducible to the bit): v_j = x_j * inv rounded once; every
// sum is serial in increasing index with fused multiply-adds and starts from
// the index-0 term; nothing else is contracted; sqrt and division are
// correctly rounded.
//
// Scheduling: the persistent design of the general band, by half-cycles:
// half 2k forms cycle k's reflector and applies it to the pivot row and the
// row segments (rows p..c-1), half 2k+1 applies it to the block and the
// column segments (rows c..ch).  Workgroups claim sweeps in increasing
// order; before half q a workgroup waits until sweep R-1 has completed
// min(q + d, all) halves (d = 2, 3, 4 for b' >= 3, 2, 1, the same lag as the
// general band, derived from the halves' footprints) and afterwards
// publishes q + 1, the final count only once R-1's is final.  Band
// accesses are agent-coherent (sc1): sweeps hand entries to workgroups on
// other XCDs, whose L2 caches are not coherent with each other.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_device.hpp"
#include "bb_internal.hpp"

namespace bb {
namespace {

__device__ __forceinline__ bool sym_wait(const uint32_t *line, uint32_t need, uint32_t limit, uint32_t *status) {
  WaitClock wc;
  while (__hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
    __builtin_amdgcn_s_sleep(1);
    if (!wc.tick(limit, status)) return false;
  }
  return true;
}

// A segment of m entries (a row at columns S or a column at rows S) in
// registers: loaded before the reflector is known, then H applied and stored.
template <typename T, int MAXM>
struct Seg {
  T a[MAXM];
  template <class B>
  __device__ __forceinline__ void load(const B &A, uint32_t o, uint32_t step, int m) {
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j < m) a[j] = A.ld_(o + uint32_t(j) * step);
  }
  // one-sided apply of H (v_0 = 1, v in LDS): s = a_0 + sum fma(a_j, v_j),
  // w = tau s, a_0 -= w, a_j = fma(-w, v_j, a_j)
  template <class B>
  __device__ __forceinline__ void apply_store(const B &A, uint32_t o, uint32_t step, const T *v, T tau, int m) {
    T s = a[0];
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (j < m) s = fma_(a[j], v[j], s);
    const T w = tau * s;
    a[0] = a[0] - w;
#pragma unroll
    for (int j = 1; j < MAXM; ++j)
      if (j < m) a[j] = fma_(-w, v[j], a[j]);
#pragma unroll
    for (int j = 0; j < MAXM; ++j)
      if (j < m) A.st_(o + uint32_t(j) * step, a[j]);
  }
};

// Row-major index of the upper-triangle element number q of an m x m block:
// (i, j), i <= j, rows in order.
__device__ __forceinline__ void tri_index(int q, int m, int &i, int &j) {
  i = 0;
  int rowlen = m;
  while (q >= rowlen) {
    q -= rowlen;
    ++i;
    --rowlen;
  }
  j = i + q;
}

template <typename T, int MAXM>
__global__ void __launch_bounds__(256) k_sym_persist(T *a, int64_t stride, int64_t n, int b, int t, int64_t nsweeps,
                                                     uint32_t *sync, uint32_t spin_limit) {
  const Band<T, kSc1> A = make_band<T, kSc1>(a, stride, 0, n);
  __shared__ T xs[MAXM], vs[MAXM], ys[MAXM], zs[MAXM];
  __shared__ T Bs[MAXM * MAXM];  // the symmetric block, both triangles
  __shared__ int64_t sR;
  __shared__ int sgo;
  uint32_t *status = sync;
  uint32_t *claim = sync + kClaim;
  uint32_t *prog = sync + kSyncHeader;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int bp = b - t;
  const int d = bp >= 3 ? 2 : (bp == 2 ? 3 : 4);  // half-cycles between consecutive sweeps
  if (tid == 0) sgo = 1;
  for (;;) {
    if (tid == 0) {
      sR = int64_t(atomicAdd(claim, 1u));
      if (launch_failed(status)) sgo = 0;  // a wait elsewhere expired: drain
    }
    __syncthreads();
    const int64_t R = sR;
    if (R >= nsweeps || !sgo) break;
    const int64_t K = cycles_of_dev(n, b, t, R);
    const int64_t Kp = R > 0 ? cycles_of_dev(n, b, t, R - 1) : 0;
    const uint32_t *pred = prog + (R - 1) * kLine;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t c = R + bp + k * b;
      const int64_t ch = c + t < n - 1 ? c + t : n - 1;
      const int m = int(ch - c + 1);
      const int64_t p = (k == 0) ? R : c - b;
      // wait for half q's predecessor progress, or publish q + 1 (every
      // wave's stores complete, then one thread moves the counter; the final
      // count waits for the predecessor's final count)
      auto wait_half = [&](int64_t q) -> bool {
        if (R > 0) {
          if (tid == 0) {
            const int64_t need = q + d < 2 * Kp ? q + d : 2 * Kp;
            sgo = sym_wait(pred, uint32_t(need), spin_limit, status);
          }
          __syncthreads();
          if (!sgo) return false;
        }
        return true;
      };
      auto publish_half = [&](int64_t q) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (tid == 0) {
          bool go = true;
          if (R > 0 && q + 1 == 2 * K) go = sym_wait(pred, uint32_t(2 * Kp), spin_limit, status);
          if (go)
            __hip_atomic_store(prog + R * kLine, uint32_t(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            sgo = 0;
        }
      };
      // half A: the reflector from the pivot row, the row segments of rows
      // p+1..c-1 (loads issued before the reflector is formed), the pivot
      // row becomes (beta, 0, ..., 0)
      if (!wait_half(2 * k)) return;
      Refl<T> h;
      {
        const int64_t nr = c - p - 1;
        Seg<T, MAXM> seg;
        const uint32_t so = tid < nr ? A.off(p + 1 + tid, c) : 0u;
        if (tid < nr) seg.load(A, so, uint32_t(sizeof(T)), m);
        if (tid < m) xs[tid] = A.ld_(A.off(p, c + tid));
        __syncthreads();
        h = house<T, MAXM, false>(xs, m);
        if (h.nz) {
          if (tid < m) vs[tid] = tid == 0 ? T(1) : xs[tid] * h.inv;
          __syncthreads();
          if (tid < nr) seg.apply_store(A, so, uint32_t(sizeof(T)), vs, h.tau, m);
        }
      }
      if (h.nz) {
        const int64_t nr = c - p - 1;
        for (int64_t r = tid + nt; r < nr; r += nt) {  // bands wider than the workgroup
          Seg<T, MAXM> more;
          const uint32_t o = A.off(p + 1 + r, c);
          more.load(A, o, uint32_t(sizeof(T)), m);
          more.apply_store(A, o, uint32_t(sizeof(T)), vs, h.tau, m);
        }
      }
      if (tid < m) {
        if (tid == 0) {
          if (h.nz) A.st_(A.off(p, c), h.beta);
        } else {
          A.st_(A.off(p, c + tid), T(0));
        }
      }
      publish_half(2 * k);
      // half B: the column segments of columns ch+1..min(ch+b, n-1) and the
      // symmetric block (staged in LDS, both triangles)
      if (!wait_half(2 * k + 1)) return;
      if (h.nz) {
        const int64_t jlast = ch + b < n - 1 ? ch + b : n - 1;
        const int64_t nc = jlast - ch;
        const int ntri = m * (m + 1) / 2;
        {
          Seg<T, MAXM> seg;
          const uint32_t so = tid < nc ? A.off(c, ch + 1 + tid) : 0u;
          if (tid < nc) seg.load(A, so, A.row_step(), m);
          for (int qq = tid; qq < ntri; qq += nt) {
            int i, j;
            tri_index(qq, m, i, j);
            const T v = A.ld_(A.off(c + i, c + j));
            Bs[i * MAXM + j] = v;
            Bs[j * MAXM + i] = v;
          }
          __syncthreads();
          if (tid < m) {  // y = tau B v, serial in j from B(i,0)
            T s = Bs[tid * MAXM];
            for (int j = 1; j < m; ++j) s = fma_(Bs[tid * MAXM + j], vs[j], s);
            ys[tid] = h.tau * s;
          }
          if (tid < nc) seg.apply_store(A, so, A.row_step(), vs, h.tau, m);
        }
        for (int64_t r = tid + nt; r < nc; r += nt) {
          Seg<T, MAXM> more;
          const uint32_t o = A.off(c, ch + 1 + r);
          more.load(A, o, A.row_step(), m);
          more.apply_store(A, o, A.row_step(), vs, h.tau, m);
        }
        __syncthreads();
        T dot = ys[0];
        for (int i = 1; i < m; ++i) dot = fma_(ys[i], vs[i], dot);
        const T alpha = -((T(0.5) * h.tau) * dot);
        if (tid < m) zs[tid] = fma_(alpha, vs[tid], ys[tid]);
        __syncthreads();
        for (int qq = tid; qq < ntri; qq += nt) {  // B -= v z^T + z v^T, upper triangle
          int i, j;
          tri_index(qq, m, i, j);
          A.st_(A.off(c + i, c + j), fma_(-vs[i], zs[j], fma_(-zs[i], vs[j], Bs[i * MAXM + j])));
        }
      }
      publish_half(2 * k + 1);
    }
    __syncthreads();  // sR is rewritten by the next claim
  }
}

// User upper rows (row i: A(i, i..i+bw), stride ld_band) -> working band,
// zero beyond bw (and past the matrix edge).
template <typename T>
__global__ void k_sym_pack(const T *__restrict__ band, int64_t ld_band, int64_t n, int bw, T *__restrict__ a,
                           int64_t stride) {
  const int64_t total = n * stride;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < total; q += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i = q / stride, o = q % stride;
    a[q] = (o <= bw && i + o < n) ? band[i * ld_band + o] : T(0);
  }
}

template <typename T>
__global__ void k_sym_extract(const T *__restrict__ a, int64_t stride, int64_t n, bool has_super, T *__restrict__ d,
                              T *__restrict__ e) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    d[i] = a[i * stride];
    if (e && i + 1 < n) e[i] = has_super ? a[i * stride + 1] : T(0);
  }
}

template <typename T, int MAXM>
hipError_t sym_persist_t(void *wband, const SymGeometry &g, int b, int t, int64_t nsweeps, uint32_t *sync, int grid,
                         int nt, uint32_t spin_limit, hipStream_t st) {
  hipLaunchKernelGGL((k_sym_persist<T, MAXM>), dim3(grid), dim3(nt), 0, st, static_cast<T *>(wband),
                     int64_t(g.stride), g.n, b, t, nsweeps, sync, spin_limit);
  return hipGetLastError();
}

template <typename T>
hipError_t sym_persist_d(int maxm, void *wband, const SymGeometry &g, int b, int t, int64_t nsweeps, uint32_t *sync,
                         int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  switch (maxm) {
    case 9: return sym_persist_t<T, 9>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 17: return sym_persist_t<T, 17>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 33: return sym_persist_t<T, 33>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    case 65: return sym_persist_t<T, 65>(wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
    default: return hipErrorInvalidValue;
  }
}

int blocks_for(int64_t work) {
  const int64_t b = (work + 255) / 256;
  return int(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

}  // namespace

hipError_t launch_sym_pack(const void *band, int64_t ld_band, void *wband, const SymGeometry &g, hipStream_t st) {
  const int blocks = blocks_for(g.n * g.stride);
  if (g.dtype == 0)
    hipLaunchKernelGGL(k_sym_pack<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float *>(band), ld_band,
                       g.n, g.bw, static_cast<float *>(wband), int64_t(g.stride));
  else
    hipLaunchKernelGGL(k_sym_pack<double>, dim3(blocks), dim3(256), 0, st, static_cast<const double *>(band),
                       ld_band, g.n, g.bw, static_cast<double *>(wband), int64_t(g.stride));
  return hipGetLastError();
}

hipError_t launch_sym_persist(int maxm, void *wband, const SymGeometry &g, int b, int t, int64_t nsweeps,
                              uint32_t *sync, int grid, int nt, uint32_t spin_limit, hipStream_t st) {
  return g.dtype == 0 ? sym_persist_d<float>(maxm, wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st)
                      : sym_persist_d<double>(maxm, wband, g, b, t, nsweeps, sync, grid, nt, spin_limit, st);
}

hipError_t launch_sym_extract(const void *wband, const SymGeometry &g, void *d, void *e, hipStream_t st) {
  const int blocks = blocks_for(g.n);
  const bool sup = g.W >= 1;
  if (g.dtype == 0)
    hipLaunchKernelGGL(k_sym_extract<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float *>(wband),
                       int64_t(g.stride), g.n, sup, static_cast<float *>(d), static_cast<float *>(e));
  else
    hipLaunchKernelGGL(k_sym_extract<double>, dim3(blocks), dim3(256), 0, st, static_cast<const double *>(wband),
                       int64_t(g.stride), g.n, sup, static_cast<double *>(d), static_cast<double *>(e));
  return hipGetLastError();
}

}  // namespace bb
