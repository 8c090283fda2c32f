// Measurement helper for the benchmark, not part of the layer library: a
// plain streaming read of a device buffer (16-byte loads, grid-stride, four
// loads in flight per thread); a lane writes only if its xor matches a key,
// so the loads stay.  It measures what HBM delivers to a kernel that does
// nothing but read, at a given transfer size: the floor a memory-bound kernel
// of that size can reach.  Built into its own library (libtl_probe.so).
//
//   int tlprobe_stream_read(const void* buf, int64_t bytes, uint32_t* out,
//                           int32_t blocks, hipStream_t stream);
// buf: device memory, 16-byte aligned, bytes a positive multiple of 16;
// out: uint32 [65] device memory not overlapping buf, out[0] the key;
// blocks: 1..65536 workgroups of 256 threads.  Returns 0 when the launch was
// enqueued, 1 on bad arguments (nothing launched), 2 when the launch failed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p,
                                                               int64_t n16,
                                                               uint32_t* __restrict__ out) {
    uint32_t acc = 0;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // the loads must stay: a lane stores only when its value matches the
    // caller's key (no workgroup-wide reduction or barrier, which cost a
    // read-only kernel several microseconds at these sizes)
    if (acc == out[0]) out[1 + (blockIdx.x & 63)] = acc;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int tlprobe_stream_read(
    const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(buf), o = reinterpret_cast<uintptr_t>(out);
    if (!buf || !out || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > 65536 ||
        (b & 15u) || (o & 3u) || (o < b + uintptr_t(bytes) && b < o + 65 * 4))
        return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(buf), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
