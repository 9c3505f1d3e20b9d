// Internal interface between the C ABI (bb_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bb_plan.hpp"

namespace bb {

hipError_t launch_pack(const void *band, int64_t ld_band, void *wband, const Geometry &g, hipStream_t st);
hipError_t launch_extract(const void *wband, const Geometry &g, void *d, void *e, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, int64_t count, uint32_t v, hipStream_t st);

// One-launch-per-step scheduler: launches nblk workgroups of nt threads for
// sweeps Rlo .. Rlo+nblk-1 of step L (cycle k = L - s R each).
hipError_t launch_step(int maxm, void *wband, const Geometry &g, int b, int t, int64_t L, int s, int64_t Rlo,
                       int64_t nblk, int nt, hipStream_t st);

}  // namespace bb
