// Scratch memory of the allocation-free attention entry point: the split
// partials live in a file-scope device array instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` (kScratchBytes)
// until the process ends.  In host code the array's name is only a stand-in
// for the symbol, never a device address: its address on the device current
// at the time comes from hipGetSymbolAddress, taken once per device and kept,
// and only that address is handed to kernels.  Every call on one GPU shares
// the array, so calls that overlap on one GPU (different streams, or threads)
// race on it; the partials need no clearing, as each split writes its whole
// record before the merge reads it.
#include <mutex>

#include "common.h"

namespace smla {
namespace {

constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    // the symbol's address on `dev` needs `dev` current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace smla
