// Device scratch owned by the library, one buffer per (device, stream): a
// block of u32 counters that are zero whenever no launch using them runs,
// followed by scratch bytes (fp32 partial sums of the K-split reductions).
// Calls on one stream are ordered by it, so the kernels of both calls share
// the stream's buffer; calls on different streams never share one.
//
// Growth allocates a larger buffer and keeps the old one until the process
// ends: a graph captured earlier on the stream still holds the old address.
// Allocation is refused while the stream is being captured.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "svdq_internal.h"

namespace svdq {
namespace {

struct Buffer {
  void* ptr = nullptr;
  size_t counters = 0;  // capacity, in u32 counters (zero-filled at allocation)
  size_t bytes = 0;     // scratch capacity after the counters
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Buffer> g_buf;
std::vector<void*> g_retired;

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

hipError_t stream_workspace(hipStream_t stream, size_t counters, size_t bytes, uint32_t** counter_ptr,
                            void** scratch_ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  Buffer& b = g_buf[{dev, stream}];
  if (b.counters < counters || b.bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    const size_t nc = std::max({counters + counters / 4, b.counters, (size_t)256});
    const size_t nb = std::max(bytes + bytes / 4, b.bytes);
    void* p = nullptr;
    e = hipMalloc(&p, round256(nc * 4) + nb);
    if (e != hipSuccess) return e;
    e = hipMemsetAsync(p, 0, round256(nc * 4), stream);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return e;
    }
    if (b.ptr) g_retired.push_back(b.ptr);
    b = Buffer{p, nc, nb};
  }
  *counter_ptr = static_cast<uint32_t*>(b.ptr);
  *scratch_ptr = static_cast<uint8_t*>(b.ptr) + round256(b.counters * 4);
  return hipSuccess;
}

}  // namespace svdq
