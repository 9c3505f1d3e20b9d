// Bandwidth probes for the memory level that holds a working band: used by
// the bench to give the cycle kernels' roofline a measured ceiling.
//
//   k_probe_stream:  z[i] = x[i] + y[i] over fp32 arrays, 16-byte vector
//                    accesses with the cycle kernels' agent-coherent cache
//                    policy; 12 bytes per element (read x, read y, write z).
//   k_probe_tadd:    B = A + A^T for an m x m fp32 matrix (the row-and-column
//                    access pattern of the page "Accelerating Bidiagonalization
//                    of Banded Matrices through Memory-Aware Bulge-Chasing on
//                    GPUs", profiling section, where a cuBLAS geam of this
//                    form is the reference point), through 64 x 64 LDS tiles
//                    so that both reads are coalesced; 12 bytes per element.
//
//   k_probe_norm:    the latency of one reflector norm (the sum of squares
//                    of the m - 1 entries below the pivot) in one wave, by
//                    the serial FMA chain the reduction uses (every lane the
//                    same entries) or by a DPP cross-lane reduction (one
//                    entry per lane, then a broadcast): a chain of `reps`
//                    dependent norms timed with the shader clock.
//
// Both bandwidth probes repeat the whole operation `reps` times in one launch, so that launch
// cost weighs nothing at cache-sized footprints and a small footprint still
// fills the chip: the work is cut into chunks (256 vectors; one 64 x 64
// tile), the (repetition, chunk) pairs are dealt to the workgroups in turn,
// and repetitions run concurrently, so a line is read by workgroups on
// several XCDs within one launch, as the band's rows are when they pass from
// one sweep group to the next.  Every repetition writes the same values: the
// results do not depend on `reps`.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb.h"
#include "bb_device.hpp"

namespace bb {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_probe_stream(const float *x, const float *y, float *z, int64_t n4,
                                                     int32_t reps) {
  const int bytes = int(uint32_t(n4 * 16));  // < 2 GiB, checked by the caller
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), 0, bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(y), 0, bytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(z, 0, bytes, kRsrcWord3);
  const int64_t chunks = (n4 + 255) / 256, items = chunks * reps;
  for (int64_t q = blockIdx.x; q < items; q += gridDim.x) {
    const int64_t i = (q % chunks) * 256 + threadIdx.x;
    if (i < n4) {
      const uint32_t o = uint32_t(i * 16);
      const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, kSc1));
      const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ry, o, 0, kSc1));
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a + b), rz, o, 0, kSc1);
    }
  }
}

constexpr int kTile = 64;

__global__ void __launch_bounds__(256) k_probe_tadd(const float *a, float *b, int32_t m, int32_t reps) {
  __shared__ float t[kTile][kTile + 1];
  const int32_t tiles = (m + kTile - 1) / kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
  const int64_t nt = int64_t(tiles) * tiles, items = nt * reps;
  for (int64_t q = blockIdx.x; q < items; q += gridDim.x) {
    const int32_t bi = int32_t((q % nt) / tiles), bj = int32_t(q % tiles);
    // stage the transposed tile A(bj-block, bi-block) in LDS
    for (int r = ty; r < kTile; r += 4) {
      const int32_t i = bj * kTile + r, j = bi * kTile + tx;
      t[r][tx] = (i < m && j < m) ? a[int64_t(i) * m + j] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < kTile; r += 4) {
      const int32_t i = bi * kTile + r, j = bj * kTile + tx;
      if (i < m && j < m) b[int64_t(i) * m + j] = a[int64_t(i) * m + j] + t[tx][r];
    }
    __syncthreads();
  }
}

template <int M>
__global__ void __launch_bounds__(64) k_probe_norm(const float *x, float *out, int32_t reps, int32_t mode,
                                                   unsigned long long *clocks) {
  const int lane = threadIdx.x;
  float v[M];
#pragma unroll
  for (int j = 0; j < M; ++j) v[j] = x[j];
  float mine = lane < M ? x[lane] : 0.f;
  float acc = 0.f;
  const uint64_t t0 = clock64();
  if (mode == 0) {
    for (int32_t r = 0; r < reps; ++r) {
      float s = v[1] * v[1];
#pragma unroll
      for (int j = 2; j < M; ++j) s = __builtin_fmaf(v[j], v[j], s);
      acc += s;
      v[1] = v[1] + s * 1e-30f;  // the next norm depends on this one
    }
  } else {
    for (int32_t r = 0; r < reps; ++r) {
      float s = lane >= 1 ? mine * mine : 0.f;
      // pairs, quads, rows of 16 (rotations), then rows into lane 63
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x124, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x128, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x142, 0xA, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x143, 0xC, 0xF, false));
      s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63));
      acc += s;
      mine = mine + s * 1e-30f;
    }
  }
  const uint64_t t1 = clock64();
  if (lane == 0) *clocks = t1 - t0;
  out[lane] = acc;
}

}  // namespace
}  // namespace bb

extern "C" {

bb_status bb_probe_norm_clocks(int32_t m, int32_t mode, int32_t reps, const void *x, void *out, void *clocks,
                               void *stream) {
  if ((m != 17 && m != 33) || (mode != 0 && mode != 1) || reps < 1 || !x || !out || !clocks) return BB_ERR_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (m == 17)
    hipLaunchKernelGGL(bb::k_probe_norm<17>, dim3(1), dim3(64), 0, st, static_cast<const float *>(x),
                       static_cast<float *>(out), reps, mode, static_cast<unsigned long long *>(clocks));
  else
    hipLaunchKernelGGL(bb::k_probe_norm<33>, dim3(1), dim3(64), 0, st, static_cast<const float *>(x),
                       static_cast<float *>(out), reps, mode, static_cast<unsigned long long *>(clocks));
  return hipGetLastError() == hipSuccess ? BB_OK : BB_ERR_HIP;
}

bb_status bb_probe_stream(const void *x, const void *y, void *z, int64_t n, int32_t reps, void *stream) {
  if (!x || !y || !z || n < 0 || (n & 3) || n * int64_t(sizeof(float)) >= (int64_t(1) << 31) || reps < 1 ||
      ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(z)) & 15))
    return BB_ERR_ARG;
  if (n == 0) return BB_OK;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    cus = 256;
  const int64_t items = (n / 4 + 255) / 256 * reps;
  const unsigned grid = unsigned(items < int64_t(cus) * 16 ? items : int64_t(cus) * 16);
  hipLaunchKernelGGL(bb::k_probe_stream, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const float *>(x), static_cast<const float *>(y), static_cast<float *>(z), n / 4,
                     reps);
  return hipGetLastError() == hipSuccess ? BB_OK : BB_ERR_HIP;
}

bb_status bb_probe_transpose_add(const void *a, void *b, int32_t m, int32_t reps, void *stream) {
  if (!a || !b || a == b || m < 0 || int64_t(m) * m > (int64_t(1) << 30) || reps < 1) return BB_ERR_ARG;
  if (m == 0) return BB_OK;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    cus = 256;
  const int64_t tiles = int64_t(m + 63) / 64, items = tiles * tiles * reps;
  const unsigned grid = unsigned(items < int64_t(cus) * 8 ? items : int64_t(cus) * 8);
  hipLaunchKernelGGL(bb::k_probe_tadd, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const float *>(a), static_cast<float *>(b), m, reps);
  return hipGetLastError() == hipSuccess ? BB_OK : BB_ERR_HIP;
}

}  // extern "C"
