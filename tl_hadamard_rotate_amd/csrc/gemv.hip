// Ternary g128 matrix-vector product on rotated activations:
//   y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[m, k]
// Products of a code in {-1, 0, 1} with an activation are exact (the multiply
// reduces to add / subtract / skip: page "Ternary Bonsai 2 27B", section
// "Что такое тернарная модель"); each 128-group is summed in fp32 and scaled
// once by its binary16 scale (page "A 27-billion model that fits in 8.6 GB",
// paragraph 2).
//
// Baseline kernel: one wave per weight row, lanes stride over the row's
// groups, fixed reduction order (bitwise deterministic).
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxTok = 16;

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemv_simple_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m0, int mt, int64_t n, int64_t k,
    void* __restrict__ y, int y_f16) {
    const int lane = threadIdx.x & 63;
    const int64_t row = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (row >= n) return;
    const int64_t groups = k / kGroup;
    const int64_t row_bytes = FMT == 0 ? groups * kTrit5GroupBytes : k / 4;
    const uint8_t* prow = packed + row * row_bytes;
    const __half* xh = reinterpret_cast<const __half*>(x) + m0 * k;

    float acc[kMaxTok];
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) acc[t] = 0.0f;

    for (int64_t g = lane; g < groups; g += 64) {
        float part[kMaxTok];
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t) part[t] = 0.0f;
        const int64_t kbase = g * kGroup;
        if (FMT == 0) {
            const uint8_t* p = prow + g * kTrit5GroupBytes;
            for (int j = 0; j < kTrit5GroupBytes; ++j) {
                uint32_t v = p[j];
                const int cnt = j < 25 ? 5 : 3;
                for (int i = 0; i < cnt; ++i) {
                    const uint32_t qd = v / 3u;
                    const int code = int(v - 3u * qd) - 1;
                    v = qd;
                    const int64_t kk = kbase + 5 * j + i;
#pragma unroll
                    for (int t = 0; t < kMaxTok; ++t)
                        if (t < mt) part[t] += float(code) * __half2float(xh[t * k + kk]);
                }
            }
        } else {
            const uint8_t* p = prow + g * (kGroup / 4);
            for (int j = 0; j < kGroup / 4; ++j) {
                const uint32_t v = p[j];
                for (int i = 0; i < 4; ++i) {
                    const int code = int((v >> (2 * i)) & 3u) - 1;
                    const int64_t kk = kbase + 4 * j + i;
#pragma unroll
                    for (int t = 0; t < kMaxTok; ++t)
                        if (t < mt) part[t] += float(code) * __half2float(xh[t * k + kk]);
                }
            }
        }
        const float s = __half2float(reinterpret_cast<const __half*>(scales)[row * groups + g]);
#pragma unroll
        for (int t = 0; t < kMaxTok; ++t) acc[t] += s * part[t];
    }
#pragma unroll
    for (int t = 0; t < kMaxTok; ++t) {
        float v = acc[t];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        acc[t] = v;
    }
    if (lane == 0) {
        for (int t = 0; t < mt; ++t) {
            const int64_t o = (m0 + t) * n + row;
            if (y_f16)
                reinterpret_cast<__half*>(y)[o] = __float2half_rn(acc[t]);
            else
                reinterpret_cast<float*>(y)[o] = acc[t];
        }
    }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    if (fmt == 1 && gemv_m1_slot2_fits(m, n, k))
        return launch_gemv_m1_slot2(packed, scales, x, n, k, y, y_f16, stream);
    if (fmt == 1) return launch_gemv_slot2(packed, scales, x, m, n, k, y, y_f16, stream);
    if (fmt == 0) return launch_gemv_trit5(packed, scales, x, m, n, k, y, y_f16, stream);
    if (fmt == 2) return launch_gemv_bit1(packed, scales, x, m, n, k, y, y_f16, stream);
    const unsigned grid = unsigned((n + kWaves - 1) / kWaves);
    for (int64_t m0 = 0; m0 < m; m0 += kMaxTok) {
        const int mt = int(m - m0 < kMaxTok ? m - m0 : kMaxTok);
        if (fmt == 0)
            hipLaunchKernelGGL(gemv_simple_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, packed,
                               scales, x, m0, mt, n, k, y, y_f16);
        else
            hipLaunchKernelGGL(gemv_simple_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, packed,
                               scales, x, m0, mt, n, k, y, y_f16);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tl
