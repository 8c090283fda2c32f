// Per-device facts the launchers need: the compute-unit count (which sizes
// every grid) and the dynamic-LDS limit of each kernel.  Both are properties
// of a device that never change while the process runs, so they are looked up
// once per device and kept; the look-ups are thread-safe.
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kMaxCached = 64;             // devices with a cached CU count
std::atomic<int> g_cus[kMaxCached];        // 0 = not looked up yet
std::mutex g_attr_mutex;
std::set<std::pair<const void*, int>> g_attr_done;   // (kernel, device)

int query_cus(int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;   // MI355X
    return n;
}

}  // namespace

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev < 0 || dev >= kMaxCached) return query_cus(dev);
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        n = query_cus(dev);
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t allow_lds(const void* kernel, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_attr_mutex);
    if (g_attr_done.count({kernel, dev})) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) g_attr_done.insert({kernel, dev});
    return e;
}

}  // namespace tl
