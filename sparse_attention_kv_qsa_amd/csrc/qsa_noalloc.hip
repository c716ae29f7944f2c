// Allocation-free device scratch for qsa_block_select_noalloc.
//
// Callers that cannot call hipMalloc (code under HIP graph capture, tight
// serving loops, harnesses that forbid it) get the same kernels with their
// scratch in one fixed array per GPU: a file-scope device variable, created
// with the code object and held until the process ends.  Its size covers
// every call qsa_block_select accepts: the few-row top-k publishes at most
// kWideMaxWordsPerRow 8-byte words per row for at most kWideMaxRows rows, and
// larger batches need no scratch.
//
// In host code `scratch` names a host-side stand-in, not the device memory:
// its device address is looked up once per device with hipGetSymbolAddress
// (which allocates nothing) while that device is current, and only that
// address is handed to kernels.  Every call on a GPU shares the array, so
// calls that overlap on one GPU race; the kernels fully rewrite the words
// they read in every call, so nothing has to start at zero.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qsa_internal.h"

namespace qsa {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t static_scratch(hipStream_t stream, size_t bytes, void **ptr) {
  *ptr = nullptr;
  if (bytes > kNoAllocScratchBytes) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = stream_device(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace qsa
