// Library-owned decode workspace, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): a file-scope device array of TQ_STATIC_WORKSPACE_BYTES,
// of which each GPU the library runs on holds its own copy until the process
// ends.  In host code the array's name only stands in for it; its device
// address, which differs per GPU, is looked up once per device with
// hipGetSymbolAddress and kept here.  Every decode call that uses it shares
// it, so such calls must not overlap on one GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tq_internal.h"

namespace tqi {
namespace {

static __device__ __align__(256) uint8_t scratch[TQ_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

}  // namespace

int static_workspace(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
      if (e != hipSuccess) return e;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace tqi
