// tl_gemm for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the same
// kernels and launch plan as tl_gemm, with the workspace taken from a
// file-scope device array instead of an argument.
//
// Every GPU the library runs on holds its own copy of `scratch` for as long as
// the process lives.  Host code never passes `scratch` itself to a kernel (in
// host code the name stands for a host-side shadow, not a device address): the
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Nothing in the
// scratch has to start at zero: the 2-bit-slot rewrite of the weights and
// every K-split part overwrite all of their bytes before they are read.  All
// calls on one GPU share its copy, so calls that may run at the same time on
// one GPU (other streams or threads) race.
#include <mutex>

#include "../../include/tl.h"
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int64_t kScratchBytes = int64_t(TL_GEMM_NOALLOC_MAX_WORKSPACE);
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out, int64_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace tl
