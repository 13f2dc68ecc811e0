// Record path around the guided kernels: a ring of pinned host slots fed by
// device-to-host copies on a dedicated stream, and the gather of a finished
// request's pages of a paged record (e.g. the FP4 KV cache) into one
// contiguous buffer.
//
// Paper: "TRACE: Rollout-Guided Quantization-Aware Training for FP4
// Reinforcement Learning of MoE Language Models", §3.2 "Motivation" (the
// records are cached during generation and moved to the training side; the
// transfer volume is what the compact record cuts) and "Key Design" (records
// indexed by trajectory, token and site; KV guidance already lives in the FP4
// KV cache).
//
// The ring is host code over the HIP runtime: one copy stream per ring at the
// default priority, one event per slot, pinned memory from hipHostMalloc. A
// push orders its copies after the work already enqueued on the producer's
// stream (an event the copy stream waits on), so the producer never blocks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/trace_fp4.h"
#include "trace_fp4_internal.h"

struct trace_ring {
  std::mutex mu;
  int device = -1;
  int64_t slot_bytes = 0;
  int32_t slots = 0;
  uint8_t* host = nullptr;
  hipStream_t copy = nullptr;
  hipEvent_t ready = nullptr;           // recorded on the producer stream at each push
  std::vector<hipEvent_t> done;         // copies of a slot finished
  std::vector<int> state;               // kFree, kInFlight, kDone
  std::vector<int64_t> used;            // bytes held by a slot
  int32_t next = 0;
};

namespace {

constexpr int kFree = 0, kInFlight = 1, kDone = 2;
constexpr int64_t kMaxRingBytes = (int64_t)1 << 40;
constexpr int32_t kMaxSlots = 4096;
constexpr int64_t kMaxGatherBytes = (int64_t)1 << 46;

int current_gfx950(int* dev) {
  const int st = tfp4::check_device();
  if (st != TRACE_OK) return st;
  return hipGetDevice(dev) == hipSuccess ? TRACE_OK : TRACE_EDEVICE;
}

void free_ring(trace_ring* r) {
  for (hipEvent_t e : r->done)
    if (e) (void)hipEventDestroy(e);
  if (r->ready) (void)hipEventDestroy(r->ready);
  if (r->copy) (void)hipStreamDestroy(r->copy);
  if (r->host) (void)hipHostFree(r->host);
  delete r;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// out page i = pool page ids[i]; ids outside [0, pool_pages) give zero bytes
// and are counted in *bad (if given). W = 16 moves uint4 words (pages and
// both bases 16-byte aligned), W = 1 single bytes.
template <int W>
__global__ __launch_bounds__(256) void gather_pages_kernel(const uint8_t* __restrict__ pool,
                                                           int64_t pool_pages, int64_t page_bytes,
                                                           const int32_t* __restrict__ ids, int64_t n,
                                                           uint8_t* __restrict__ out, uint32_t* bad) {
  const int64_t wpp = page_bytes / W;                    // words per page
  const int64_t total = n * wpp;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += stride) {
    const int64_t i = w / wpp, o = w - i * wpp;
    const int64_t id = ids[i];
    const bool ok = id >= 0 && id < pool_pages;
    if constexpr (W == 16) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = reinterpret_cast<const uint4*>(pool)[id * wpp + o];
      reinterpret_cast<uint4*>(out)[w] = v;
    } else {
      out[w] = ok ? pool[id * page_bytes + o] : (uint8_t)0;
    }
    if (!ok && o == 0 && bad != nullptr) atomicAdd(bad, 1u);
  }
}

}  // namespace

extern "C" {

int trace_ring_create(int64_t slot_bytes, int32_t slots, trace_ring** out) {
  if (out == nullptr) return TRACE_EINVAL;
  *out = nullptr;
  if (slot_bytes <= 0 || slots <= 0 || slots > kMaxSlots) return TRACE_ESHAPE;
  if (slot_bytes > kMaxRingBytes / slots) return TRACE_ESHAPE;
  int dev = -1;
  int st = current_gfx950(&dev);
  if (st != TRACE_OK) return st;
  trace_ring* r = new (std::nothrow) trace_ring();
  if (r == nullptr) return TRACE_ELAUNCH;
  r->device = dev;
  r->slot_bytes = slot_bytes;
  r->slots = slots;
  r->done.assign(slots, nullptr);
  r->state.assign(slots, kFree);
  r->used.assign(slots, 0);
  bool ok = hipHostMalloc((void**)&r->host, (size_t)(slot_bytes * slots), hipHostMallocDefault) == hipSuccess;
  ok = ok && hipStreamCreateWithFlags(&r->copy, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&r->ready, hipEventDisableTiming) == hipSuccess;
  for (int32_t i = 0; ok && i < slots; ++i)
    ok = hipEventCreateWithFlags(&r->done[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    free_ring(r);
    return TRACE_ELAUNCH;
  }
  *out = r;
  return TRACE_OK;
}

int trace_ring_destroy(trace_ring* r) {
  if (r == nullptr) return TRACE_EINVAL;
  const bool ok = hipStreamSynchronize(r->copy) == hipSuccess;
  free_ring(r);
  return ok ? TRACE_OK : TRACE_ELAUNCH;
}

int trace_ring_push(trace_ring* r, const void* const* srcs, const int64_t* bytes, int32_t n,
                    void* after_stream, int32_t* slot_out) {
  if (r == nullptr || slot_out == nullptr || n <= 0 || srcs == nullptr || bytes == nullptr)
    return TRACE_EINVAL;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (bytes[i] < 0) return TRACE_ESHAPE;
    if (bytes[i] > 0 && srcs[i] == nullptr) return TRACE_EINVAL;
    total += bytes[i];
    if (total > r->slot_bytes) return TRACE_ESHAPE;
  }
  std::lock_guard<std::mutex> lock(r->mu);
  const int32_t s = r->next;
  if (r->state[s] != kFree) return TRACE_EBUSY;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != r->device) return TRACE_EDEVICE;
  if (hipEventRecord(r->ready, static_cast<hipStream_t>(after_stream)) != hipSuccess ||
      hipStreamWaitEvent(r->copy, r->ready, 0) != hipSuccess)
    return TRACE_ELAUNCH;
  uint8_t* dst = r->host + (int64_t)s * r->slot_bytes;
  for (int32_t i = 0; i < n; ++i) {
    if (bytes[i] == 0) continue;
    if (hipMemcpyAsync(dst, srcs[i], (size_t)bytes[i], hipMemcpyDeviceToHost, r->copy) != hipSuccess)
      return TRACE_ELAUNCH;
    dst += bytes[i];
  }
  if (hipEventRecord(r->done[s], r->copy) != hipSuccess) return TRACE_ELAUNCH;
  r->state[s] = kInFlight;
  r->used[s] = total;
  r->next = (s + 1) % r->slots;
  *slot_out = s;
  return TRACE_OK;
}

int trace_ring_wait(trace_ring* r, int32_t slot) {
  if (r == nullptr || slot < 0 || slot >= r->slots) return TRACE_EINVAL;
  hipEvent_t e;
  {
    std::lock_guard<std::mutex> lock(r->mu);
    if (r->state[slot] == kFree) return TRACE_EINVAL;
    if (r->state[slot] == kDone) return TRACE_OK;
    e = r->done[slot];
  }
  if (hipEventSynchronize(e) != hipSuccess) return TRACE_ELAUNCH;
  std::lock_guard<std::mutex> lock(r->mu);
  r->state[slot] = kDone;
  return TRACE_OK;
}

int trace_ring_query(trace_ring* r, int32_t slot) {
  if (r == nullptr || slot < 0 || slot >= r->slots) return TRACE_EINVAL;
  std::lock_guard<std::mutex> lock(r->mu);
  if (r->state[slot] == kFree) return TRACE_EINVAL;
  if (r->state[slot] == kDone) return 1;
  const hipError_t q = hipEventQuery(r->done[slot]);
  if (q == hipSuccess) {
    r->state[slot] = kDone;
    return 1;
  }
  return q == hipErrorNotReady ? 0 : TRACE_ELAUNCH;
}

const void* trace_ring_slot(trace_ring* r, int32_t slot, int64_t* bytes_out) {
  if (r == nullptr || slot < 0 || slot >= r->slots) return nullptr;
  std::lock_guard<std::mutex> lock(r->mu);
  if (r->state[slot] != kDone) return nullptr;
  if (bytes_out != nullptr) *bytes_out = r->used[slot];
  return r->host + (int64_t)slot * r->slot_bytes;
}

int trace_ring_release(trace_ring* r, int32_t slot) {
  if (r == nullptr || slot < 0 || slot >= r->slots) return TRACE_EINVAL;
  std::lock_guard<std::mutex> lock(r->mu);
  if (r->state[slot] != kDone) return TRACE_EINVAL;
  r->state[slot] = kFree;
  r->used[slot] = 0;
  return TRACE_OK;
}

int trace_gather_pages(const uint8_t* pool, int64_t pool_pages, int64_t page_bytes,
                       const int32_t* page_ids, int64_t n, uint8_t* out, uint32_t* bad_ids,
                       void* stream) {
  if (pool_pages < 0 || page_bytes <= 0 || n < 0) return TRACE_ESHAPE;
  if (n > 0 && page_bytes > kMaxGatherBytes / n) return TRACE_ESHAPE;
  if (pool_pages > 0 && page_bytes > kMaxGatherBytes / pool_pages) return TRACE_ESHAPE;
  if (n > 0 && (page_ids == nullptr || out == nullptr || (pool_pages > 0 && pool == nullptr)))
    return TRACE_EINVAL;
  if (((uintptr_t)page_ids & 3u) != 0 || ((uintptr_t)bad_ids & 3u) != 0) return TRACE_EALIGN;
  const int64_t out_bytes = n * page_bytes;
  if (overlaps(out, out_bytes, pool, pool_pages * page_bytes) ||
      overlaps(out, out_bytes, page_ids, 4 * n) || overlaps(out, out_bytes, bad_ids, 4) ||
      overlaps(bad_ids, 4, pool, pool_pages * page_bytes) || overlaps(bad_ids, 4, page_ids, 4 * n))
    return TRACE_EALIAS;
  int dev = -1;
  int st = current_gfx950(&dev);
  if (st != TRACE_OK) return st;
  if (n == 0) return TRACE_OK;
  const bool wide = page_bytes % 16 == 0 && ((uintptr_t)pool & 15u) == 0 && ((uintptr_t)out & 15u) == 0;
  const int64_t words = wide ? out_bytes / 16 : out_bytes;
  int64_t blocks = (words + 256 * 4 - 1) / (256 * 4);
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  void* argv[] = {(void*)&pool, (void*)&pool_pages, (void*)&page_bytes, (void*)&page_ids,
                  (void*)&n, (void*)&out, (void*)&bad_ids};
  const void* k = wide ? reinterpret_cast<const void*>(&gather_pages_kernel<16>)
                       : reinterpret_cast<const void*>(&gather_pages_kernel<1>);
  return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(256), argv, 0, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? TRACE_OK
             : TRACE_ELAUNCH;
}

}  // extern "C"
