// Measurement references beside the path's kernels: plain streams of 16-byte
// words with the same access policy (nontemporal loads and stores, 256
// threads of 4 words per workgroup tile: the fastest of 256 or 512 threads
// and 2 to 16 words measured), one stream in and one out (a copy)
// or two in and one out (the read/write mix of the fused guided pass, which
// reads the training and rollout tensors and writes y). They compute nothing
// of the method; the benchmark times them on the same device, in the same
// run, as the HBM rates the kernels are compared with.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/trace_fp4.h"
#include "trace_fp4_internal.h"

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamWords = 4;                        // 16-byte words per thread
constexpr int64_t kStreamTile = (int64_t)kStreamThreads * kStreamWords;
constexpr int64_t kMaxStreamBytes = (int64_t)1 << 37;   // 2^23 workgroups, 2^31 work-items at most

typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));

// out[i] = a[i] (TWO false) or a[i] ^ b[i] (TWO true), words [0, words).
template <bool TWO>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const v4u_t* __restrict__ a,
                                                                const v4u_t* __restrict__ b,
                                                                v4u_t* __restrict__ out, int64_t words) {
  const int64_t base = (int64_t)blockIdx.x * kStreamTile + threadIdx.x;
  v4u_t v[kStreamWords], w[kStreamWords];
#pragma unroll
  for (int j = 0; j < kStreamWords; ++j) {
    const int64_t i = base + (int64_t)j * kStreamThreads;
    if (i < words) {
      v[j] = __builtin_nontemporal_load(a + i);
      if constexpr (TWO) w[j] = __builtin_nontemporal_load(b + i);
    }
  }
#pragma unroll
  for (int j = 0; j < kStreamWords; ++j) {
    const int64_t i = base + (int64_t)j * kStreamThreads;
    if (i < words) {
      v4u_t r = v[j];
      if constexpr (TWO) r ^= w[j];
      __builtin_nontemporal_store(r, out + i);
    }
  }
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int run_stream(const void* a, const void* b, void* out, int64_t bytes, void* stream) {
  const bool two = b != nullptr;
  if (bytes < 0 || bytes > kMaxStreamBytes || bytes % 16 != 0) return TRACE_ESHAPE;
  if (bytes > 0 && (a == nullptr || out == nullptr)) return TRACE_EINVAL;
  if (((uintptr_t)a & 15u) != 0 || ((uintptr_t)b & 15u) != 0 || ((uintptr_t)out & 15u) != 0) return TRACE_EALIGN;
  if (overlap(out, bytes, a, bytes) || (two && overlap(out, bytes, b, bytes))) return TRACE_EALIAS;
  const int st = tfp4::check_device();
  if (st != TRACE_OK) return st;
  if (bytes == 0) return TRACE_OK;
  const int64_t words = bytes / 16;
  const int64_t blocks = (words + kStreamTile - 1) / kStreamTile;
  const v4u_t* pa = static_cast<const v4u_t*>(a);
  const v4u_t* pb = static_cast<const v4u_t*>(b);
  v4u_t* po = static_cast<v4u_t*>(out);
  void* argv[] = {(void*)&pa, (void*)&pb, (void*)&po, (void*)&words};
  const void* k = two ? reinterpret_cast<const void*>(&stream_kernel<true>)
                      : reinterpret_cast<const void*>(&stream_kernel<false>);
  return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kStreamThreads), argv, 0, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? TRACE_OK
             : TRACE_ELAUNCH;
}

}  // namespace

extern "C" {

int trace_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (src == nullptr && bytes > 0) return TRACE_EINVAL;
  return run_stream(src, nullptr, dst, bytes, stream);
}

int trace_stream_mix(const void* a, const void* b, void* out, int64_t bytes, void* stream) {
  if ((a == nullptr || b == nullptr) && bytes > 0) return TRACE_EINVAL;
  return run_stream(a, b, out, bytes, stream);
}

}  // extern "C"
