// Device scratch owned by the library.
//
// Some launches need a few bytes to megabytes of device memory beyond the
// caller's inputs and outputs (the published group words of the few-row
// top-k and of the fused decode select, the chunk partials of the decode
// attention).  They come from one buffer per (device,
// stream): work enqueued on one stream runs in order, so consecutive calls on
// a stream can reuse the same bytes, and calls on different streams never
// share them.  A buffer only grows; a buffer that is outgrown is kept (not
// freed) until the process ends, because work still queued on the stream may
// be using it and freeing it would force a synchronisation.
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

hipError_t workspace(hipStream_t stream, size_t bytes, void **ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mutex);
  Buffer &b = g_buffers[{dev, stream}];
  if (b.bytes < bytes) {
    // Grow geometrically (at least 1 MiB) so a sequence of growing calls
    // allocates O(log) times.
    size_t want = bytes < (size_t(1) << 20) ? (size_t(1) << 20) : bytes;
    if (want < 2 * b.bytes) want = 2 * b.bytes;
    void *p = nullptr;
    e = hipMalloc(&p, want);
    if (e != hipSuccess) return e;
    if (b.ptr) g_retired.push_back(b.ptr);
    b.ptr = p;
    b.bytes = want;
  }
  *ptr = b.ptr;
  return hipSuccess;
}

}  // namespace qsa
