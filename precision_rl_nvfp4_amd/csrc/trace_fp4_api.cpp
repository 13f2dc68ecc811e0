// C ABI of the rollout-guided FP4 library: argument validation on the host,
// then kernel launches on the caller's stream. The operations and their
// sources in the paper are documented in include/trace_fp4.h.
//
// Validation order: (1) scalars (fmt, bits, flags, sizes), (2) NULL checks,
// (3) alignment, (4) aliasing of outputs against every other buffer, (5) the
// current device must be gfx950. Steps 1-4 make no HIP call, so every error
// path short of EDEVICE is testable on a machine without a GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/trace_fp4.h"
#include "trace_fp4_internal.h"

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
bool any_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int block_of(int fmt) { return fmt == TRACE_FMT_NVFP4 ? 16 : 32; }

bool valid_fmt(int fmt) { return fmt == TRACE_FMT_NVFP4 || fmt == TRACE_FMT_MXFP4; }

// N = rows * cols with cols % B == 0 and no overflow; the limit keeps every
// byte offset (2N) and unit index inside int64 with room to spare.
int shape_n(int fmt, int64_t rows, int64_t cols, int64_t* n) {
  if (rows < 0 || cols < 0) return TRACE_ESHAPE;
  if (cols % block_of(fmt) != 0) return TRACE_ESHAPE;
  const int64_t kMaxElems = (int64_t)1 << 50;
  if (cols != 0 && rows > kMaxElems / cols) return TRACE_ESHAPE;
  *n = rows * cols;
  return TRACE_OK;
}

// Per-device result of the gfx950 check: 0 unknown, 1 yes, 2 no.
std::atomic<int> g_dev_ok[64];

int check_device() {
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

int launched(hipError_t e) { return e == hipSuccess ? TRACE_OK : TRACE_ELAUNCH; }

// Checks shared by quantize_rtn and encode_guidance. `plane_bytes` is the
// size of the code or bit plane.
int check_rtn_args(int fmt, int64_t n, const uint16_t* x, const float* gin, const uint8_t* plane,
                   int64_t plane_bytes, uint32_t plane_align, const uint8_t* scales,
                   const float* gout, const uint16_t* y) {
  if (fmt == TRACE_FMT_NVFP4) {
    if ((gin == nullptr) == (gout == nullptr)) return TRACE_EINVAL;
  } else if (gin != nullptr || gout != nullptr) {
    return TRACE_EINVAL;
  }
  if (n > 0 && (x == nullptr || plane == nullptr || scales == nullptr)) return TRACE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(plane, plane_align) || !aligned(gin, 4) ||
      !aligned(gout, 4))
    return TRACE_EALIGN;
  const Range ins[] = {{x, 2 * n}, {gin, 4}};
  const Range outs[] = {{plane, plane_bytes}, {scales, n / block_of(fmt)}, {gout, 8}, {y, 2 * n}};
  if (any_alias(outs, 4, ins, 2)) return TRACE_EALIAS;
  return TRACE_OK;
}

int run_rtn(int fmt, int plane_mode, int64_t n, const uint16_t* x, const float* gin, uint8_t* plane,
            uint8_t* scales, float* gout, uint16_t* y, void* stream) {
  int st = check_device();
  if (st != TRACE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t units = n / tfp4::kUnitElems;
  if (fmt == TRACE_FMT_NVFP4 && gout != nullptr) {
    hipError_t e = tfp4::launch_global_scale(x, units, gout, s);
    if (e != hipSuccess) return TRACE_ELAUNCH;
    return launched(tfp4::launch_quantize(fmt, plane_mode, true, x, units, gout, plane, scales, y, s));
  }
  return launched(tfp4::launch_quantize(fmt, plane_mode, false, x, units, const_cast<float*>(gin),
                                        plane, scales, y, s));
}

// Checks shared by decode_guidance and guided_fake_quant.
int check_train_args(int fmt, int64_t n, const uint16_t* x, const uint8_t* guide, int64_t guide_bytes,
                     uint32_t guide_align, bool guide_needed, const uint8_t* scales,
                     const float* gscale) {
  if (fmt == TRACE_FMT_NVFP4) {
    if (gscale == nullptr) return TRACE_EINVAL;
  } else if (gscale != nullptr) {
    return TRACE_EINVAL;
  }
  if (!guide_needed && guide != nullptr) return TRACE_EINVAL;
  if (n > 0 && (x == nullptr || scales == nullptr || (guide_needed && guide == nullptr)))
    return TRACE_EINVAL;
  if (!aligned(x, 16) || !aligned(guide, guide_align) || !aligned(gscale, 4)) return TRACE_EALIGN;
  (void)guide_bytes;
  return TRACE_OK;
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
    default: return "unknown status";
  }
}

int quantize_rtn(int fmt, int64_t rows, int64_t cols, const uint16_t* x, const float* gscale_in,
                 uint8_t* codes, uint8_t* scales, float* gscale_out, uint16_t* y_opt, void* stream) {
  if (!valid_fmt(fmt)) return TRACE_EINVAL;
  int64_t n = 0;
  int st = shape_n(fmt, rows, cols, &n);
  if (st != TRACE_OK) return st;
  st = check_rtn_args(fmt, n, x, gscale_in, codes, n / 2, 4, scales, gscale_out, y_opt);
  if (st != TRACE_OK) return st;
  return run_rtn(fmt, 0, n, x, gscale_in, codes, scales, gscale_out, y_opt, stream);
}

int encode_guidance(int fmt, int bits, int64_t rows, int64_t cols, const uint16_t* x_rollout,
                    const float* gscale_in, uint8_t* guide, uint8_t* scales, float* gscale_out,
                    uint16_t* y_rollout_opt, void* stream) {
  if (!valid_fmt(fmt) || (bits != 1 && bits != 4)) return TRACE_EINVAL;
  int64_t n = 0;
  int st = shape_n(fmt, rows, cols, &n);
  if (st != TRACE_OK) return st;
  const int64_t gbytes = bits == 1 ? n / 8 : n / 2;
  st = check_rtn_args(fmt, n, x_rollout, gscale_in, guide, gbytes, bits == 1 ? 1 : 4, scales,
                      gscale_out, y_rollout_opt);
  if (st != TRACE_OK) return st;
  return run_rtn(fmt, bits == 1 ? 1 : 0, n, x_rollout, gscale_in, guide, scales, gscale_out,
                 y_rollout_opt, stream);
}

int decode_guidance(int fmt, int64_t rows, int64_t cols, const uint16_t* x_train,
                    const uint8_t* mbits, const uint8_t* scales, const float* gscale,
                    uint8_t* ref_codes, void* stream) {
  if (!valid_fmt(fmt)) return TRACE_EINVAL;
  int64_t n = 0;
  int st = shape_n(fmt, rows, cols, &n);
  if (st != TRACE_OK) return st;
  st = check_train_args(fmt, n, x_train, mbits, n / 8, 1, true, scales, gscale);
  if (st != TRACE_OK) return st;
  if (n > 0 && ref_codes == nullptr) return TRACE_EINVAL;
  if (!aligned(ref_codes, 4)) return TRACE_EALIGN;
  const Range ins[] = {{x_train, 2 * n}, {mbits, n / 8}, {scales, n / block_of(fmt)}, {gscale, 4}};
  const Range outs[] = {{ref_codes, n / 2}};
  if (any_alias(outs, 1, ins, 4)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_guided(fmt, 1, true, x_train, n / tfp4::kUnitElems, mbits, scales,
                                      gscale, nullptr, ref_codes, static_cast<hipStream_t>(stream)));
}

int guided_fake_quant(int fmt, int bits, int64_t rows, int64_t cols, const uint16_t* x_train,
                      const uint8_t* guide, const uint8_t* scales, const float* gscale, uint16_t* y,
                      uint8_t* codes_opt, void* stream) {
  if (!valid_fmt(fmt) || (bits != 0 && bits != 1 && bits != 4)) return TRACE_EINVAL;
  int64_t n = 0;
  int st = shape_n(fmt, rows, cols, &n);
  if (st != TRACE_OK) return st;
  const int64_t gbytes = bits == 1 ? n / 8 : bits == 4 ? n / 2 : 0;
  st = check_train_args(fmt, n, x_train, guide, gbytes, bits == 4 ? 4 : 1, bits != 0, scales, gscale);
  if (st != TRACE_OK) return st;
  if (n > 0 && y == nullptr) return TRACE_EINVAL;
  if (!aligned(y, 16) || !aligned(codes_opt, 4)) return TRACE_EALIGN;
  const Range ins[] = {{x_train, 2 * n}, {guide, gbytes}, {scales, n / block_of(fmt)}, {gscale, 4}};
  const Range outs[] = {{y, 2 * n}, {codes_opt, n / 2}};
  if (any_alias(outs, 2, ins, 4)) return TRACE_EALIAS;
  st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_guided(fmt, bits, false, x_train, n / tfp4::kUnitElems, guide,
                                      scales, gscale, y, codes_opt,
                                      static_cast<hipStream_t>(stream)));
}

int64_t trace_stats_workspace_bytes(int64_t n) {
  if (n < 0) return 0;
  return 2 * (int64_t)sizeof(double) * tfp4::stats_groups(n);
}

int discrepancy_stats(int64_t n, const uint16_t* x_t, const uint16_t* x_r, const uint16_t* y_t,
                      const uint16_t* y_r, double* acc3, int accumulate, void* work,
                      int64_t work_bytes, void* stream) {
  if (accumulate != 0 && accumulate != 1) return TRACE_EINVAL;
  if (n < 0 || n > ((int64_t)1 << 50)) return TRACE_ESHAPE;
  if (acc3 == nullptr || work == nullptr) return TRACE_EINVAL;
  if (n > 0 && (x_t == nullptr || x_r == nullptr || y_t == nullptr || y_r == nullptr))
    return TRACE_EINVAL;
  if (work_bytes < trace_stats_workspace_bytes(n)) return TRACE_ESHAPE;
  if (!aligned(x_t, 16) || !aligned(x_r, 16) || !aligned(y_t, 16) || !aligned(y_r, 16) ||
      !aligned(acc3, 8) || !aligned(work, 8))
    return TRACE_EALIGN;
  const Range ins[] = {{x_t, 2 * n}, {x_r, 2 * n}, {y_t, 2 * n}, {y_r, 2 * n}};
  const Range outs[] = {{acc3, 24}, {work, work_bytes}};
  if (any_alias(outs, 2, ins, 4)) return TRACE_EALIAS;
  int st = check_device();
  if (st != TRACE_OK) return st;
  return launched(tfp4::launch_stats(n, x_t, x_r, y_t, y_r, acc3, accumulate,
                                     static_cast<double*>(work), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
