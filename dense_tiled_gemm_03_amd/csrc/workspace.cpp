// Device scratch for kernels that combine partial results of several
// workgroups (the split-K skinny and tile kernels): one buffer per (device,
// stream), allocated on first use, grown on demand and kept until the
// process ends.  A buffer that has been outgrown is retired, not freed: a
// graph captured on the stream may still hold kernels that use it, and
// replaying such a graph must not touch freed memory.  Each growth at least
// doubles the size, so the retired buffers of a stream add up to less than
// its current one.
//
// Contract with the kernels: the first kWorkspaceCounterBytes of the buffer
// (the completion counters) are zero whenever a kernel that uses them
// starts, and every such kernel leaves them zero when it ends; partial
// results live only past that area, so a call with few counters and large
// partials never leaves data where a later call with more counters looks.
// A fresh buffer is cleared on the stream before any kernel runs on it.
// Work on one stream is ordered, so calls on one stream never share the
// buffer at the same time; each stream has its own buffer.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "common.hpp"

namespace tg {
namespace {

struct Buffer {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_mutex;
std::map<std::pair<int, hipStream_t>, Buffer>& buffers() {
  static auto* m = new std::map<std::pair<int, hipStream_t>, Buffer>();  // never destroyed
  return *m;
}

}  // namespace

void* stream_workspace(hipStream_t stream, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  Buffer& b = buffers()[{dev, stream}];
  if (b.bytes >= bytes) return b.ptr;
  // Allocation is not allowed while the stream is being captured into a graph:
  // the caller then runs its variant that needs no scratch.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return nullptr;
  // whole MiB, at least twice the buffer it replaces; the old one stays
  // allocated (earlier kernels or captured graphs may still use it)
  size_t want = (bytes + 0xFFFFF) & ~size_t(0xFFFFF);
  if (want < 2 * b.bytes) want = 2 * b.bytes;
  void* p = nullptr;
  if (hipMalloc(&p, want) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipMemsetAsync(p, 0, want, stream) != hipSuccess) {
    (void)hipFree(p);
    return nullptr;
  }
  b.ptr = p;  // the outgrown buffer, if any, is retired: never freed
  b.bytes = want;
  return p;
}

}  // namespace tg
