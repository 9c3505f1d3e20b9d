// Device-side building blocks shared by the kernels of the band -> bidiagonal
// reduction: the Householder reflector under the arithmetic contract, the
// band accessor through a buffer resource, and the geometry of one cycle.
//
// Arithmetic contract (so that results are reproducible to the bit by any
// implementation following it): reflector H = I - tau v v^T with
// v = (1, x_j / (alpha - beta)), beta = -sign(alpha) ||x|| (sign(+-0) = +1),
// tau = (beta - alpha) / beta; the tail sum of squares and every dot product
// are serial in increasing index with fused multiply-adds, nothing else is
// contracted (-ffp-contract=off), square root and division are correctly
// rounded.  A zero tail makes the reflector the identity; the annihilated
// entries are written as exact zeros either way.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bb {
namespace {

// s_waitcnt immediate with vmcnt = 0 and expcnt / lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float sqrt_(float a) { return __builtin_sqrtf(a); }
__device__ __forceinline__ double sqrt_(double a) { return __builtin_sqrt(a); }
__device__ __forceinline__ float div_(float a, float b) { return a / b; }
__device__ __forceinline__ double div_(double a, double b) { return a / b; }
// Half precision: fma is the fp16 instruction (one rounding); sqrt and
// division are the correctly rounded fp32 operations rounded once to fp16,
// which equals the correctly rounded fp16 result (24 >= 2*11 + 2 bits).  The
// empty asm keeps the compiler from rewriting the fp32 operation into its own
// fp16 sequence.
__device__ __forceinline__ _Float16 fma_(_Float16 a, _Float16 b, _Float16 c) { return __builtin_fmaf16(a, b, c); }
__device__ __forceinline__ _Float16 sqrt_(_Float16 a) {
  float r = __builtin_sqrtf(float(a));
  asm volatile("" : "+v"(r));
  return _Float16(r);
}
__device__ __forceinline__ _Float16 div_(_Float16 a, _Float16 b) {
  float q = float(a) / float(b);
  asm volatile("" : "+v"(q));
  return _Float16(q);
}

// Bounded waits.  Every poll loop calls WaitClock::tick once per poll;
// once per `every` polls (a power of two) it reads the 100 MHz constant
// clock (wall_clock64: 10 ns per tick) and, with `global`, the launch's
// status word.  The wait expires `limit` ticks after its first such check,
// or, with `global`, as soon as any other wait of the launch has expired
// (the status word is nonzero); on expiry it sets the status word.  Waits
// that poll memory and the idle loops of the group kernel's auxiliary waves
// read the status word (a memory round trip, off their critical path); the
// sweeps' LDS waits check only the clock and their group's abort flag, which
// the auxiliary waves raise.  Workgroups also read the status word when they
// claim work, so after a first expiry the whole launch drains within about
// one limit: a chain of waits cannot outlast it.
// The clock is read in its low 32 bits (42.9 s before it wraps), so a bound
// stays below 2^31 ticks (21.4 s).
struct WaitClock {
  uint32_t polls = 0;
  uint32_t t0 = 0;
  // false: expired (the status word is set)
  template <uint32_t every = 16, bool global = true>
  __device__ __forceinline__ bool tick(uint32_t limit, uint32_t *status) {
    static_assert((every & (every - 1)) == 0, "power of two");
    if ((++polls & (every - 1)) != 0) return true;
    const uint32_t now = uint32_t(wall_clock64());
    if (polls == every) {
      t0 = now;
      return true;
    }
    if (now - t0 <= limit && (!global || __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0))
      return true;
    __hip_atomic_store(status, uint32_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
};

__device__ __forceinline__ bool launch_failed(const uint32_t *status) {
  return __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

template <typename T>
struct Refl {
  T beta, tau, inv;
  bool nz;  // false: identity (zero tail)
};

// Reflector of x[0..m-1] (x in LDS, read by every thread: broadcast).
// FULL: m == MAXM, no bounds on the loop.
template <typename T, int MAXM, bool FULL>
__device__ __forceinline__ Refl<T> house(const T *x, int m) {
  Refl<T> h;
  const T alpha = x[0];
  T s = T(0);
#pragma unroll
  for (int j = 1; j < MAXM; ++j)
    if (FULL || j < m) s = fma_(x[j], x[j], s);
  if (s == T(0)) {
    h.nz = false;
    h.beta = alpha;
    h.tau = T(0);
    h.inv = T(0);
    return h;
  }
  const T nrm = sqrt_(fma_(alpha, alpha, s));
  h.beta = (alpha >= T(0)) ? -nrm : nrm;
  h.tau = div_(h.beta - alpha, h.beta);
  h.inv = div_(T(1), alpha - h.beta);
  h.nz = true;
  return h;
}

// Band in memory through a buffer resource: element (i, j) at byte offset
// (i*ld + j - i + sub) * sizeof(T).  Out-of-range loads return zero and
// out-of-range stores are dropped by the hardware.  AUX is the cache policy:
// 0 for ordinary accesses (one launch per step: the kernel boundary orders
// the cycles), kSc1 for agent-scope accesses that stay coherent across the
// XCDs' separate L2 caches (workgroups handing data to each other inside one
// launch).
constexpr int kSc1 = 16;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer descriptor

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int AUX>
struct Band {
  __amdgpu_buffer_rsrc_t r;
  int64_t ld;
  int32_t sub;
  int64_t n;
  __device__ __forceinline__ uint32_t off(int64_t i, int64_t j) const {
    return uint32_t((i * ld + (j - i + sub)) * int64_t(sizeof(T)));
  }
  // byte offset of (i, j) and byte strides: next column +sizeof(T), next row
  // (same column) +(ld-1)*sizeof(T)
  __device__ __forceinline__ uint32_t row_step() const { return uint32_t((ld - 1) * int64_t(sizeof(T))); }
  __device__ __forceinline__ T ld_(uint32_t o) const {
    if constexpr (sizeof(T) == 2)
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, AUX));
    else if constexpr (sizeof(T) == 4)
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, AUX));
    else
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, AUX));
  }
  __device__ __forceinline__ u32x4 ld4_(uint32_t o) const { return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, AUX); }
  __device__ __forceinline__ void st4_(uint32_t o, u32x4 v) const { __builtin_amdgcn_raw_buffer_store_b128(v, r, o, 0, AUX); }
  __device__ __forceinline__ void st_(uint32_t o, T v) const {
    if constexpr (sizeof(T) == 2)
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, o, 0, AUX);
    else if constexpr (sizeof(T) == 4)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, o, 0, AUX);
    else
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, o, 0, AUX);
  }
};

template <typename T, int AUX>
__device__ __forceinline__ Band<T, AUX> make_band(T *a, int64_t ld, int32_t sub, int64_t n) {
  Band<T, AUX> B;
  B.r = __builtin_amdgcn_make_buffer_rsrc(a, 0, int(uint32_t(n * ld * int64_t(sizeof(T)))), kRsrcWord3);
  B.ld = ld;
  B.sub = sub;
  B.n = n;
  return B;
}

// Geometry of cycle (R, k) of the pass (b, t).
struct Cyc {
  int64_t c, ch, r, jend;
  int m;
  __device__ __forceinline__ Cyc(int64_t n, int b, int t, int64_t R, int64_t k) {
    c = R + (b - t) + k * b;
    ch = c + t < n - 1 ? c + t : n - 1;
    m = int(ch - c + 1);
    r = (k == 0) ? R : c - b;
    jend = c + t + b < n - 1 ? c + t + b : n - 1;
  }
};

// Cycles of sweep R: k = 0 .. K-1 with R + b' + k b <= n-2.
__device__ __forceinline__ int64_t cycles_of_dev(int64_t n, int b, int t, int64_t R) {
  const int64_t last = n - 2 - R - (b - t);
  return last < 0 ? 0 : last / b + 1;
}

}  // namespace
}  // namespace bb
