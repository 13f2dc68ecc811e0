// Internal interface between the C-ABI layer (trace_fp4_api.cpp) and the
// kernels (trace_fp4_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfp4 {

// Element counts handled per thread step: one 16-byte load of 8 bf16.
constexpr int kUnitElems = 8;
constexpr int kThreads = 256;

// Upper bound on the partial sums of discrepancy_stats (one per workgroup).
constexpr int kStatsMaxGroups = 1024;

int64_t stats_groups(int64_t n);

// Every launcher enqueues on `stream` and returns the first HIP error seen.
// Sizes are already validated; `units` = N / 8.

// Global amax -> gscale_out = {S, A}. `x` may be NULL when units == 0.
hipError_t launch_global_scale(const uint16_t* x, int64_t units, float* gscale_out,
                               hipStream_t stream);

// Quantize (RTN) one tensor: fmt 0 NVFP4 / 1 MXFP4; plane_mode 0 = code
// plane (u8[N/2]), 1 = mantissa-bit plane (u8[N/8]). `gsrc` is the device
// float holding S (NVFP4; NULL for MXFP4); when `s_from_amax` is set, gsrc
// points at gscale_out, S is derived from gsrc[1] = A, and gsrc[0] gets S.
hipError_t launch_quantize(int fmt, int plane_mode, bool s_from_amax, const uint16_t* x,
                           int64_t units, float* gsrc, uint8_t* plane, uint8_t* scales,
                           uint16_t* y, hipStream_t stream);

// Guided rounding / Reconstruct under the rollout scales. bits in {0, 1, 4};
// decode_only writes reference codes (bits must be 1) into `codes` and no y.
hipError_t launch_guided(int fmt, int bits, bool decode_only, const uint16_t* x,
                         int64_t units, const uint8_t* guide, const uint8_t* scales,
                         const float* gscale, uint16_t* y, uint8_t* codes,
                         hipStream_t stream);

// Deterministic float64 sums into acc3; `partials` holds 2 * stats_groups(n) doubles.
hipError_t launch_stats(int64_t n, const uint16_t* xt, const uint16_t* xr, const uint16_t* yt,
                        const uint16_t* yr, double* acc3, int accumulate, double* partials,
                        hipStream_t stream);

}  // namespace tfp4
