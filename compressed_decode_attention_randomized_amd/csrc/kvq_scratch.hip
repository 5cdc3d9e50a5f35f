// The fixed device scratch of kvq_decode_noalloc: the split partials of one
// decode call, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, one copy per GPU the library runs
// on, held until the process ends.  Host code never passes the array's name
// to a kernel (in host code it is only a stand-in for the symbol): the first
// call on each device resolves that device's copy with hipGetSymbolAddress,
// with the device current, and every later call uses the pointer kept here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace kvq
