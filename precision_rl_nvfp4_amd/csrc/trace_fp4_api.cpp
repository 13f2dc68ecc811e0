// C ABI of the rollout-guided FP4 library: argument validation on the host,
// then kernel launches on the caller's stream. The operations and their
// sources in the paper are documented in include/trace_fp4.h.
//
// Validation order: (1) scalars (fmt, bits, flags, sizes, grouping), (2) NULL
// checks, (3) workspace sizes, (4) alignment, (5) aliasing of outputs against
// every other buffer, (6) the current device must be gfx950. Steps 1-5 make
// no HIP call, so every error path short of EDEVICE is testable on a machine
// without a GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/trace_fp4.h"
#include "trace_fp4_internal.h"

static_assert(TRACE_MISMATCH_COUNTS == tfp4::kMismatchCounts, "mismatch count layout");
static_assert(TRACE_NOALLOC_SCRATCH_BYTES == tfp4::kScratchBytes, "scratch size");

namespace {

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlaps(const Range& a, const Range& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes <= 0 || b.bytes <= 0) return false;
  uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Every output must be disjoint from every input and from the other outputs.
template <int NO, int NI>
bool any_alias(const Range (&outs)[NO], const Range (&ins)[NI]) {
  for (int i = 0; i < NO; ++i) {
    for (int j = 0; j < NI; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < NO; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int block_of(int fmt) { return fmt == TRACE_FMT_NVFP4 ? 16 : 32; }

bool valid_fmt(int fmt) { return fmt == TRACE_FMT_NVFP4 || fmt == TRACE_FMT_MXFP4; }

constexpr int64_t kMaxOffsetGroups = (int64_t)1 << 22;  // row-offset groups per call

// Guidance planes: bits 1..3 keep the low bits of each magnitude index (N*bits/8
// bytes), 4 the full codes (N/2). Units of 8 elements are read whole, so a
// plane is aligned to one unit's bytes when that is a power of two.
int64_t guide_bytes(int bits, int64_t n) { return n * bits / 8; }
uintptr_t guide_align(int bits) { return bits == 4 ? 4 : bits == 2 ? 2 : 1; }

// A validated call shape: N elements in G groups of upg units.
struct CallShape {
  int64_t n;
  tfp4::Shape sh;
};

// N = rows * cols with cols % B == 0, group_rows dividing rows, N at most
// 2^35 and G * (tiles + kPartMax) below 2^31 (tiles of kTileUnits units per
// group). Together they bound every launch: the guided pass's 1024-unit tiles
// number at most 2^22 + G <= 2^22 + 2^21 workgroups of 512 threads, below the
// 2^32 work-items a dispatch packet can describe, and the quantize and amax
// launches less.
int shape_of(int fmt, int64_t rows, int64_t cols, int64_t group_rows, CallShape* out) {
  if (rows < 0 || cols < 0 || group_rows < 0) return TRACE_ESHAPE;
  if (cols % block_of(fmt) != 0) return TRACE_ESHAPE;
  if (group_rows > 0 && rows % group_rows != 0) return TRACE_ESHAPE;
  const int64_t kMaxElems = (int64_t)1 << 35;
  if (cols != 0 && rows > kMaxElems / cols) return TRACE_ESHAPE;
  const int64_t grows = group_rows > 0 ? group_rows : rows;
  out->n = rows * cols;
  out->sh.groups = group_rows > 0 ? rows / group_rows : 1;
  out->sh.upg = grows * cols / tfp4::kUnitElems;
  // A launch holds up to G tiles per group plus G amax workgroups per group.
  const int64_t tiles = (out->sh.upg + tfp4::kTileUnits - 1) / tfp4::kTileUnits;
  if (out->sh.groups > 0 && tiles + tfp4::kPartMax > INT32_MAX / out->sh.groups) return TRACE_ESHAPE;
  return TRACE_OK;
}

// Per-device result of the gfx950 check: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[64];

}  // namespace

int tfp4::check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TRACE_EDEVICE;
  if (dev < 64) {
    int c = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return TRACE_OK;
    if (c == 2) return TRACE_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TRACE_EDEVICE;
  bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? TRACE_OK : TRACE_EDEVICE;
}

namespace {

using tfp4::check_device;

int launched(hipError_t e) { return e == hipSuccess ? TRACE_OK : TRACE_ELAUNCH; }

// Shared by quantize_rtn, encode_guidance and encode_guidance_noalloc.
// `plane_bits` gives the size and alignment of the code or bit plane. With
// use_scratch the workspace is the library's own device array instead of
// `work` (which is then ignored), up to tfp4::kScratchBytes.
int run_rtn(int fmt, int plane_bits, int64_t rows, int64_t cols, int64_t group_rows,
            const uint16_t* x, const float* gin, uint8_t* plane, uint8_t* scales, float* gout,
            uint16_t* y, void* work, int64_t work_bytes, void* stream, bool use_scratch = false) {
  CallShape cs;
  int st = shape_of(fmt, rows, cols, group_rows, &cs);
  if (st != TRACE_OK) return st;
  const int64_t n = cs.n, G = cs.sh.groups;
  if (fmt == TRACE_FMT_NVFP4) {
    if ((gin == nullptr) == (gout == nullptr)) return TRACE_EINVAL;
  } else if (gin != nullptr || gout != nullptr) {
    return TRACE_EINVAL;
  }
  if (n > 0 && (x == nullptr || plane == nullptr || scales == nullptr)) return TRACE_EINVAL;
  const int64_t wneed = gout != nullptr && n > 0 ? tfp4::quant_work_bytes(fmt, cs.sh) : 0;
  const bool need_work = wneed > 0;
  if (use_scratch) {
    work = nullptr;
    if (wneed > tfp4::kScratchBytes) return TRACE_ESHAPE;
  } else {
    if (need_work && work == nullptr) return TRACE_EINVAL;
    if (work_bytes < wneed) return TRACE_ESHAPE;
  }
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(plane, guide_align(plane_bits)) ||
      !aligned(gin, 4) ||
      !aligned(gout, 4) || (need_work && !aligned(work, 8)))
    return TRACE_EALIGN;
  const Range ins[] = {{x, 2 * n}, {gin, 8 * G}};
  const Range outs[] = {{plane, guide_bytes(plane_bits, n)}, {scales, n / block_of(fmt)}, {gout, 8 * G},
                        {y, 2 * n}, {need_work ? work : nullptr, wneed}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  if (use_scratch && need_work && tfp4::scratch_of_current_device(&work) != hipSuccess) return TRACE_ELAUNCH;
  return launched(tfp4::launch_quantize(fmt, plane_bits, cs.sh, x, gin, gout, plane, scales, y,
                                        need_work ? work : nullptr,
                                        static_cast<hipStream_t>(stream)));
}

// Checks shared by the training-side calls: scales, gscale, guide.
int check_train(int fmt, int64_t n, const uint16_t* x, const uint8_t* guide, bool guide_needed,
                const uint8_t* scales, const float* gscale) {
  if (fmt == TRACE_FMT_NVFP4) {
    if (gscale == nullptr) return TRACE_EINVAL;
  } else if (gscale != nullptr) {
    return TRACE_EINVAL;
  }
  if (!guide_needed && guide != nullptr) return TRACE_EINVAL;
  if (n > 0 && (x == nullptr || scales == nullptr || (guide_needed && guide == nullptr)))
    return TRACE_EINVAL;
  return TRACE_OK;
}

int run_guided(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
               const uint16_t* x, const uint16_t* xr, bool stats, const uint8_t* guide,
               const uint8_t* scales, const float* gscale, uint16_t* y, uint8_t* codes,
               double* acc3, int64_t* counts, int accumulate, void* work, int64_t work_bytes,
               void* stream) {
  if (!valid_fmt(fmt) || bits < 0 || bits > 4) return TRACE_EINVAL;
  if (stats && accumulate != 0 && accumulate != 1) return TRACE_EINVAL;
  CallShape cs;
  int st = shape_of(fmt, rows, cols, group_rows, &cs);
  if (st != TRACE_OK) return st;
  const int64_t n = cs.n, G = cs.sh.groups;
  st = check_train(fmt, n, x, guide, bits != 0, scales, gscale);
  if (st != TRACE_OK) return st;
  if (n > 0 && y == nullptr) return TRACE_EINVAL;
  int64_t wneed = 0;
  if (stats) {
    if (acc3 == nullptr || (n > 0 && xr == nullptr)) return TRACE_EINVAL;
    wneed = n > 0 ? tfp4::guided_stats_work_bytes(fmt, cs.sh) : 0;
    if (wneed > 0 && work == nullptr) return TRACE_EINVAL;
    if (work_bytes < wneed) return TRACE_ESHAPE;
  }
  if (!aligned(x, 16) || !aligned(xr, 16) || !aligned(y, 16) || !aligned(codes, 4) ||
      !aligned(guide, guide_align(bits)) || !aligned(gscale, 4) || !aligned(acc3, 8) ||
      !aligned(counts, 8) || (wneed > 0 && !aligned(work, 8)))
    return TRACE_EALIGN;
  const int64_t gbytes = guide_bytes(bits, n);
  const Range ins[] = {{x, 2 * n}, {xr, stats ? 2 * n : 0}, {guide, gbytes},
                       {scales, n / block_of(fmt)}, {gscale, 8 * G}};
  const Range outs[] = {{y, 2 * n}, {codes, n / 2}, {acc3, stats ? 24 : 0},
                        {counts, stats ? 8 * (int64_t)TRACE_MISMATCH_COUNTS : 0},
                        {wneed > 0 ? work : nullptr, wneed}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_guided(fmt, bits, false, cs.sh, x, guide, scales, gscale, y, codes,
                                      stats ? xr : nullptr, stats ? acc3 : nullptr,
                                      stats ? counts : nullptr, accumulate,
                                      wneed > 0 ? work : nullptr, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int trace_abi_version(void) { return TRACE_ABI_VERSION; }

const char* trace_status_str(int status) {
  switch (status) {
    case TRACE_OK: return "TRACE_OK";
    case TRACE_EINVAL: return "TRACE_EINVAL";
    case TRACE_ESHAPE: return "TRACE_ESHAPE";
    case TRACE_EALIGN: return "TRACE_EALIGN";
    case TRACE_EALIAS: return "TRACE_EALIAS";
    case TRACE_EDEVICE: return "TRACE_EDEVICE";
    case TRACE_ELAUNCH: return "TRACE_ELAUNCH";
    case TRACE_EBUSY: return "TRACE_EBUSY";
    default: return "unknown status";
  }
}

int64_t trace_set_encode_batch(int64_t groups_per_batch) {
  if (groups_per_batch < 0) return TRACE_EINVAL;
  return tfp4::set_encode_batch(groups_per_batch);
}

int64_t trace_set_wait_limit(int64_t polls) {
  if (polls < 0 || polls > INT32_MAX) return TRACE_EINVAL;
  return tfp4::set_wait_limit(polls);
}

int trace_encode_wait_failures(uint64_t* count) {
  if (count == nullptr) return TRACE_EINVAL;
  const int st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::read_wait_failures(count));
}

int64_t trace_quant_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t group_rows) {
  if (!valid_fmt(fmt)) return -1;
  CallShape cs;
  if (shape_of(fmt, rows, cols, group_rows, &cs) != TRACE_OK) return -1;
  return tfp4::quant_work_bytes(fmt, cs.sh);
}

int64_t trace_guided_stats_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t group_rows) {
  if (!valid_fmt(fmt)) return -1;
  CallShape cs;
  if (shape_of(fmt, rows, cols, group_rows, &cs) != TRACE_OK) return -1;
  return tfp4::guided_stats_work_bytes(fmt, cs.sh);
}

int64_t trace_stats_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return tfp4::stats_work_bytes(n);
}

int64_t trace_grouped_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t groups) {
  if (!valid_fmt(fmt)) return -1;
  CallShape cs;
  if (shape_of(fmt, rows, cols, 0, &cs) != TRACE_OK || groups < 1 || groups > kMaxOffsetGroups) return -1;
  if (fmt == TRACE_FMT_MXFP4) return 0;
  return tfp4::offs_work_bytes(rows, cols, groups);
}

int quantize_rtn(int fmt, int64_t rows, int64_t cols, int64_t group_rows, const uint16_t* x,
                 const float* gscale_in, uint8_t* codes, uint8_t* scales, float* gscale_out,
                 uint16_t* y_opt, void* work, int64_t work_bytes, void* stream) {
  if (!valid_fmt(fmt)) return TRACE_EINVAL;
  return run_rtn(fmt, 4, rows, cols, group_rows, x, gscale_in, codes, scales, gscale_out, y_opt,
                 work, work_bytes, stream);
}

int encode_guidance(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                    const uint16_t* x_rollout, const float* gscale_in, uint8_t* guide,
                    uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* work,
                    int64_t work_bytes, void* stream) {
  if (!valid_fmt(fmt) || bits < 1 || bits > 4) return TRACE_EINVAL;
  return run_rtn(fmt, bits, rows, cols, group_rows, x_rollout, gscale_in, guide, scales,
                 gscale_out, y_rollout_opt, work, work_bytes, stream);
}

int encode_guidance_noalloc(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                            const uint16_t* x_rollout, const float* gscale_in, uint8_t* guide,
                            uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* stream) {
  if (!valid_fmt(fmt) || bits < 1 || bits > 4) return TRACE_EINVAL;
  return run_rtn(fmt, bits, rows, cols, group_rows, x_rollout, gscale_in, guide, scales, gscale_out,
                 y_rollout_opt, nullptr, 0, stream, true);
}

int decode_guidance(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                    const uint16_t* x_train, const uint8_t* guide, const uint8_t* scales,
                    const float* gscale, uint8_t* ref_codes, void* stream) {
  if (!valid_fmt(fmt) || bits < 1 || bits > 3) return TRACE_EINVAL;
  CallShape cs;
  int st = shape_of(fmt, rows, cols, group_rows, &cs);
  if (st != TRACE_OK) return st;
  const int64_t n = cs.n, G = cs.sh.groups;
  st = check_train(fmt, n, x_train, guide, true, scales, gscale);
  if (st != TRACE_OK) return st;
  if (n > 0 && ref_codes == nullptr) return TRACE_EINVAL;
  if (!aligned(x_train, 16) || !aligned(ref_codes, 4) || !aligned(gscale, 4) ||
      !aligned(guide, guide_align(bits)))
    return TRACE_EALIGN;
  const Range ins[] = {{x_train, 2 * n}, {guide, guide_bytes(bits, n)}, {scales, n / block_of(fmt)},
                       {gscale, 8 * G}};
  const Range outs[] = {{ref_codes, n / 2}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_guided(fmt, bits, true, cs.sh, x_train, guide, scales, gscale, nullptr,
                                      ref_codes, nullptr, nullptr, nullptr, 0, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

int guided_fake_quant(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                      const uint16_t* x_train, const uint8_t* guide, const uint8_t* scales,
                      const float* gscale, uint16_t* y, uint8_t* codes_opt, void* stream) {
  return run_guided(fmt, bits, rows, cols, group_rows, x_train, nullptr, false, guide, scales,
                    gscale, y, codes_opt, nullptr, nullptr, 0, nullptr, 0, stream);
}

int guided_fake_quant_stats(int fmt, int bits, int64_t rows, int64_t cols, int64_t group_rows,
                            const uint16_t* x_train, const uint16_t* x_rollout,
                            const uint8_t* guide, const uint8_t* scales, const float* gscale,
                            uint16_t* y, uint8_t* codes_opt, double* acc3, int64_t* counts_opt,
                            int accumulate, void* work, int64_t work_bytes, void* stream) {
  return run_guided(fmt, bits, rows, cols, group_rows, x_train, x_rollout, true, guide, scales,
                    gscale, y, codes_opt, acc3, counts_opt, accumulate, work, work_bytes, stream);
}

int encode_guidance_grouped(int fmt, int bits, int64_t rows, int64_t cols, int64_t groups,
                            const int64_t* row_offsets, const uint16_t* x_rollout, uint8_t* guide,
                            uint8_t* scales, float* gscale_out, uint16_t* y_rollout_opt, void* work,
                            int64_t work_bytes, void* stream) {
  if (!valid_fmt(fmt) || bits < 1 || bits > 4) return TRACE_EINVAL;
  if (groups < 1 || groups > kMaxOffsetGroups) return TRACE_ESHAPE;
  if (row_offsets == nullptr) return TRACE_EINVAL;
  if (fmt == TRACE_FMT_MXFP4) {  // no global scale: the groups do not change anything
    if (gscale_out != nullptr) return TRACE_EINVAL;
    return run_rtn(fmt, bits, rows, cols, 0, x_rollout, nullptr, guide, scales, nullptr, y_rollout_opt,
                   nullptr, 0, stream);
  }
  CallShape cs;
  int st = shape_of(fmt, rows, cols, 0, &cs);
  if (st != TRACE_OK) return st;
  if (groups < 1 || groups > kMaxOffsetGroups) return TRACE_ESHAPE;
  const int64_t n = cs.n;
  if (row_offsets == nullptr || gscale_out == nullptr) return TRACE_EINVAL;
  if (n > 0 && (x_rollout == nullptr || guide == nullptr || scales == nullptr)) return TRACE_EINVAL;
  const int64_t wneed = tfp4::offs_work_bytes(rows, cols, groups);
  if (tfp4::offs_entries(rows, cols, groups) > INT32_MAX) return TRACE_ESHAPE;
  if (work == nullptr) return TRACE_EINVAL;
  if (work_bytes < wneed) return TRACE_ESHAPE;
  if (!aligned(x_rollout, 16) || !aligned(y_rollout_opt, 16) || !aligned(guide, guide_align(bits)) ||
      !aligned(gscale_out, 4) || !aligned(row_offsets, 8) || !aligned(work, 8))
    return TRACE_EALIGN;
  const Range ins[] = {{x_rollout, 2 * n}, {row_offsets, 8 * (groups + 1)}};
  const Range outs[] = {{guide, guide_bytes(bits, n)}, {scales, n / block_of(fmt)},
                        {gscale_out, 8 * groups}, {y_rollout_opt, 2 * n}, {work, wneed}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_encode_offsets(bits, rows, cols, groups, row_offsets, x_rollout, guide,
                                              scales, gscale_out, y_rollout_opt, work,
                                              static_cast<hipStream_t>(stream)));
}

int guided_fake_quant_grouped(int fmt, int bits, int64_t rows, int64_t cols, int64_t groups,
                              const int64_t* row_offsets, const uint16_t* x_train, const uint8_t* guide,
                              const uint8_t* scales, const float* gscale, uint16_t* y, uint8_t* codes_opt,
                              void* work, int64_t work_bytes, void* stream) {
  if (!valid_fmt(fmt) || bits < 0 || bits > 4) return TRACE_EINVAL;
  if (groups < 1 || groups > kMaxOffsetGroups) return TRACE_ESHAPE;
  if (row_offsets == nullptr) return TRACE_EINVAL;
  if (fmt == TRACE_FMT_MXFP4)
    return run_guided(fmt, bits, rows, cols, 0, x_train, nullptr, false, guide, scales, gscale, y,
                      codes_opt, nullptr, nullptr, 0, nullptr, 0, stream);
  CallShape cs;
  int st = shape_of(fmt, rows, cols, 0, &cs);
  if (st != TRACE_OK) return st;
  if (groups < 1 || groups > kMaxOffsetGroups) return TRACE_ESHAPE;
  const int64_t n = cs.n;
  st = check_train(fmt, n, x_train, guide, bits != 0, scales, gscale);
  if (st != TRACE_OK) return st;
  if (row_offsets == nullptr || (n > 0 && y == nullptr)) return TRACE_EINVAL;
  const int64_t wneed = tfp4::offs_work_bytes(rows, cols, groups);
  if (tfp4::offs_entries(rows, cols, groups) > INT32_MAX) return TRACE_ESHAPE;
  if (work == nullptr) return TRACE_EINVAL;
  if (work_bytes < wneed) return TRACE_ESHAPE;
  if (!aligned(x_train, 16) || !aligned(y, 16) || !aligned(codes_opt, 4) ||
      !aligned(guide, guide_align(bits)) || !aligned(gscale, 4) || !aligned(row_offsets, 8) ||
      !aligned(work, 8))
    return TRACE_EALIGN;
  const Range ins[] = {{x_train, 2 * n}, {guide, guide_bytes(bits, n)}, {scales, n / block_of(fmt)},
                       {gscale, 8 * groups}, {row_offsets, 8 * (groups + 1)}};
  const Range outs[] = {{y, 2 * n}, {codes_opt, n / 2}, {work, wneed}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_guided_offsets(bits, rows, cols, groups, row_offsets, x_train, guide, scales,
                                              gscale, y, codes_opt, work, static_cast<hipStream_t>(stream)));
}

int discrepancy_stats(int64_t n, const uint16_t* x_t, const uint16_t* x_r, const uint16_t* y_t,
                      const uint16_t* y_r, double* acc3, int accumulate, void* work,
                      int64_t work_bytes, void* stream) {
  if (accumulate != 0 && accumulate != 1) return TRACE_EINVAL;
  if (n < 0 || n > ((int64_t)1 << 44)) return TRACE_ESHAPE;
  if (acc3 == nullptr || work == nullptr) return TRACE_EINVAL;
  if (n > 0 && (x_t == nullptr || x_r == nullptr || y_t == nullptr || y_r == nullptr))
    return TRACE_EINVAL;
  if (work_bytes < trace_stats_workspace_bytes(n)) return TRACE_ESHAPE;
  if (!aligned(x_t, 16) || !aligned(x_r, 16) || !aligned(y_t, 16) || !aligned(y_r, 16) ||
      !aligned(acc3, 8) || !aligned(work, 8))
    return TRACE_EALIGN;
  const Range ins[] = {{x_t, 2 * n}, {x_r, 2 * n}, {y_t, 2 * n}, {y_r, 2 * n}};
  const Range outs[] = {{acc3, 24}, {work, work_bytes}};
  if (any_alias(outs, ins)) return TRACE_EALIAS;
  int st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_stats(n, x_t, x_r, y_t, y_r, acc3, accumulate,
                                     static_cast<double*>(work), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
