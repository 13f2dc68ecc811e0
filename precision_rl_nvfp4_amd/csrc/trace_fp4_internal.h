// Internal interface between the C-ABI layer (trace_fp4_api.cpp) and the
// kernels (trace_fp4_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfp4 {

// One "unit" is a 16-byte load of 8 bf16 elements.
constexpr int kUnitElems = 8;
constexpr int kThreads = 256;
// A workgroup tile: kThreads lanes x kUPT units.
constexpr int kUPT = 8;
constexpr int64_t kTileUnits = (int64_t)kThreads * kUPT;

// Amax partial maxima kept per global-scale group (one per workgroup of the
// amax pass).
constexpr int kPartMax = 1024;

// Mismatch diagnostics of guided_fake_quant_stats: two 15-bin distance
// histograms and two direction counts.
constexpr int kMismatchCounts = 32;

// Shape of one call: G groups of `upg` units each (units = G * upg), every
// group with its own FP32 global scale (NVFP4). Blocks never straddle groups.
struct Shape {
  int64_t groups;
  int64_t upg;  // units per group
};

// Workspace of quantize_rtn / encode_guidance when S comes from the amax:
// uint32 partial maxima (two passes) or tagged tile maxima (single pass)
// [groups][kPartMax], then the single pass's published S words
// [groups][1024]; none for MXFP4 or for NVFP4 groups packed several to a
// tile (their amax is reduced inside the tile).
int64_t quant_work_bytes(int fmt, const Shape& sh);
// Workspace of guided_fake_quant_stats: float64 partial sums, 2 per workgroup,
// 64 second-level pairs, and the per-workgroup mismatch counts.
int64_t guided_stats_work_bytes(int fmt, const Shape& sh);
// Workspace of discrepancy_stats.
int64_t stats_work_bytes(int64_t n);

// RTN quantization of a tensor (quantize_rtn / encode_guidance).
//   fmt 0 NVFP4 / 1 MXFP4; plane_mode = bits of the plane: 4 = code plane
//   u8[N/2], 1..3 = the low 1..3 magnitude bits, u8[N*bits/8]. NVFP4:
//   exactly one of gin (S of group g at gin[2g]) and gout (receives {S, A}
//   per group, computed from the amax) is non-NULL, and `work` holds
//   quant_work_bytes when gout is used. MXFP4: both NULL.
hipError_t launch_quantize(int fmt, int plane_mode, const Shape& sh, const uint16_t* x,
                           const float* gin, float* gout, uint8_t* plane, uint8_t* scales,
                           uint16_t* y, void* work, hipStream_t stream);

// Guided rounding under the rollout scales (guided_fake_quant, bits 0..4),
// Reconstruct alone (decode_guidance: decode_only, bits 1..3, writes
// reference codes), and
// the fused discrepancy sums (xr and acc3 non-NULL) with, when counts is also
// non-NULL, the mismatch diagnostics.
hipError_t launch_guided(int fmt, int bits, bool decode_only, const Shape& sh,
                         const uint16_t* x, const uint8_t* guide, const uint8_t* scales,
                         const float* gscale, uint16_t* y, uint8_t* codes, const uint16_t* xr,
                         double* acc3, int64_t* counts, int accumulate, void* work,
                         hipStream_t stream);

// Row-offset groups (NVFP4): groups are the row ranges [off[g], off[g + 1])
// given by a device array of G + 1 row offsets (clamped into [0, rows] and
// made nondecreasing on the device; rows outside [off[0], off[G]) are not
// touched). Workspace: offs_work_bytes; the launches use offs_entries
// workgroups (tiles of every group, plus slack of one per group).
int64_t offs_work_bytes(int64_t rows, int64_t cols, int64_t groups);
int64_t offs_entries(int64_t rows, int64_t cols, int64_t groups);
hipError_t launch_encode_offsets(int bits, int64_t rows, int64_t cols, int64_t G, const int64_t* off_in,
                                 const uint16_t* x, uint8_t* plane, uint8_t* scales, float* gout,
                                 uint16_t* y, void* work, hipStream_t stream);
hipError_t launch_guided_offsets(int bits, int64_t rows, int64_t cols, int64_t G, const int64_t* off_in,
                                 const uint16_t* x, const uint8_t* guide, const uint8_t* scales,
                                 const float* gscale, uint16_t* y, uint8_t* codes, void* work,
                                 hipStream_t stream);

// TRACE_OK when the current device is a gfx950, else TRACE_EDEVICE (cached
// per device).
int check_device();

// Groups per batch of NVFP4 encoding with scales from the amax (each launch
// quantizes one batch and reads the next for its amax); 0 = automatic.
// Returns the previous value.
int64_t set_encode_batch(int64_t groups);

// Polls after which a bounded wait of the single-pass encode gives up; 0 =
// the default. Returns the previous value.
int64_t set_wait_limit(int64_t polls);

// The current device's count of single-pass waits that gave up since the
// library was loaded (a synchronous device-to-host copy).
hipError_t read_wait_failures(uint64_t* out);

// Bytes of the library's own device scratch array (one per device), the
// workspace of encode_guidance_noalloc, and its address on the current
// device (looked up once per device; allocates nothing).
constexpr int64_t kScratchBytes = (int64_t)4 << 20;
hipError_t scratch_of_current_device(void** out);

// Deterministic float64 sums of discrepancy_stats into acc3.
hipError_t launch_stats(int64_t n, const uint16_t* xt, const uint16_t* xr, const uint16_t* yt,
                        const uint16_t* yr, double* acc3, int accumulate, double* partials,
                        hipStream_t stream);

}  // namespace tfp4
