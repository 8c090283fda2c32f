// Library-owned device workspaces: one buffer per (kind, device, stream), so
// that launches that may overlap never share one.  A buffer grows on demand
// (hipMalloc, after hipFree of the smaller one; neither can be captured into
// a HIP graph) and is never shrunk or freed before the process ends.
#include <map>
#include <mutex>
#include <tuple>

#include "tl_internal.h"

namespace tl {
namespace {

struct Buffer {
    void* p = nullptr;
    size_t bytes = 0;
};
std::mutex g_mutex;
std::map<std::tuple<int, int, hipStream_t>, Buffer> g_buffers;

}  // namespace

hipError_t workspace(int kind, hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_mutex);
    Buffer& b = g_buffers[std::make_tuple(kind, dev, stream)];
    if (b.bytes < bytes) {
        if (b.p) (void)hipFree(b.p);
        b.p = nullptr;
        b.bytes = 0;
        if ((e = hipMalloc(&b.p, bytes)) != hipSuccess) return e;
        b.bytes = bytes;
    }
    *out = b.p;
    return hipSuccess;
}

}  // namespace tl
