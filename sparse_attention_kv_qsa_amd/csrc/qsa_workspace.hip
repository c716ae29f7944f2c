// Device scratch owned by the library.
//
// Some launches need a few bytes to megabytes of device memory beyond the
// caller's inputs and outputs (the published group words of the few-row
// top-k and of the fused decode select, the chunk partials of the decode
// attention).  They come from one buffer per (device,
// stream), keyed on the device the stream belongs to: work enqueued on one
// stream runs in order, so consecutive calls on
// a stream can reuse the same bytes, and calls on different streams never
// share them.  A buffer only grows; a buffer that is outgrown is kept (not
// freed) until the process ends, because work still queued on the stream may
// be using it and freeing it would force a synchronisation.
//
// The key is the stream handle.  A stream destroyed while work that uses its
// buffer is still queued, whose handle the runtime then hands to a new
// stream, would give that new stream the same buffer while the old work may
// still run: callers synchronise a stream before destroying it.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "qsa_internal.h"

namespace qsa {
namespace {

struct Buffer {
  void *ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mutex;
std::map<std::pair<int, hipStream_t>, Buffer> g_buffers;
std::vector<void *> g_retired;  // outgrown buffers, kept for the process lifetime

}  // namespace

hipError_t stream_device(hipStream_t stream, int *dev) {
  if (stream == nullptr) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(stream, &d);
  *dev = int(d);
  return e;
}

hipError_t workspace(hipStream_t stream, size_t bytes, void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = stream_device(stream, &dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mutex);
  Buffer &b = g_buffers[{dev, stream}];
  if (b.bytes < bytes) {
    // Grow geometrically (at least 1 MiB) so a sequence of growing calls
    // allocates O(log) times.  The buffer lives on the stream's device, which
    // need not be the calling thread's current one.
    size_t want = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
    if (want < 2 * b.bytes) want = 2 * b.bytes;
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipMalloc(&p, want);
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) {
      if (p) (void)hipFree(p);
      return e;
    }
    if (b.ptr) g_retired.push_back(b.ptr);
    b.ptr = p;
    b.bytes = want;
  }
  *ptr = b.ptr;
  return hipSuccess;
}

}  // namespace qsa
