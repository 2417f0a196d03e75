// moe_forward_decode_noalloc: the decode layer with its workspace in a static
// device array instead of a caller-supplied buffer, for callers that cannot
// allocate device memory.  Same kernels, same validation, same results as
// moe_forward_decode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "moe_internal.h"

namespace bqmoe {

// The decode workspace of every call on one GPU.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code this name is
// only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call on
// that device), or nullptr if the lookup fails.
static void* scratch_ptr(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
    (void)hipGetLastError();  // leave no sticky error for the caller's next call
    return nullptr;
  }
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace bqmoe

using namespace bqmoe;

extern "C" moe_status moe_forward_decode_noalloc(const moe_layer* L, const uint16_t* x,
                                                 int32_t T, uint32_t flags, moe_routing* R,
                                                 uint16_t* out, void* stream) {
  if (!L || !R) return MOE_ERR_INVALID_ARG;
  if (T < 1 || T > MOE_MAX_DECODE_TOKENS) return MOE_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  void* ws = scratch_ptr(dev);
  if (!ws) return MOE_ERR_DEVICE;
  // decode_call rejects a layer whose decode workspace exceeds the array
  // (MOE_ERR_WORKSPACE) before anything is enqueued
  return decode_call(L, x, T, flags, R, ws, MOE_NOALLOC_SCRATCH_BYTES, out, ~0u, stream, true);
}
