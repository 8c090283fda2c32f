// Prefill ternary g128 GEMM: y[m, n] = sum_k x[m, k] * code[n, k] * S[n, k/128].
// The weight tile of each K step (one 128-group) is expanded on chip to exact
// binary16 values code * S (a code in {-1,0,1} times a binary16 scale is a
// binary16 number) and the contraction runs on fp16 matrix cores with fp32
// accumulation.  Prompt processing is the practical bottleneck the pages name
// for slower chips (page "A 27-billion model that fits in 8.6 GB", paragraph 4).
//
// Baseline tiling: 64 x 64 output tile per workgroup of 4 waves, each wave a
// 32 x 32 quadrant made of 2 x 2 v_mfma_f32_16x16x32_f16.  A and B tiles are
// stored K-contiguous in LDS with an 8-half row pad.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = 64, BN = 64, BK = kGroup;
constexpr int kLdsStride = BK + 8;   // halves per LDS row

// digit d -> binary16 bits of (d - 1) * s, with s given as binary16 bits
__device__ __forceinline__ uint16_t code_times_scale(uint32_t d, uint16_t s) {
    return d == 1u ? uint16_t(0) : (d == 0u ? uint16_t(s ^ 0x8000u) : s);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_simple_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int64_t m, int64_t n, int64_t k, void* __restrict__ y,
    int y_f16) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * kLdsStride];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t n_tiles = (n + BN - 1) / BN;
    const int64_t m_base = (int64_t(blockIdx.x) / n_tiles) * BM;
    const int64_t n_base = (int64_t(blockIdx.x) % n_tiles) * BN;
    const int64_t groups = k / kGroup;
    const int64_t row_bytes = FMT == 0 ? groups * kTrit5GroupBytes : k / 4;
    const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;

    float4v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};

    for (int64_t g = 0; g < groups; ++g) {
        // A tile: 64 rows x 128 halves; thread -> (row, 32-half chunk)
        {
            const int r = tid >> 2, c = (tid & 3) * 32;
            const int64_t gm = m_base + r;
            uint4 v[4];
            if (gm < m) {
                const uint4* src = reinterpret_cast<const uint4*>(x + gm * k + g * kGroup + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = src[i];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = uint4{0, 0, 0, 0};
            }
            uint4* dst = reinterpret_cast<uint4*>(As + r * kLdsStride + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[i] = v[i];
        }
        // B tile: 64 weight rows x 128 codes, expanded to code * scale
        {
            const int r = tid >> 2, part = tid & 3;
            const int64_t gn = n_base + r;
            uint16_t* dst = Bs + r * kLdsStride;
            if (gn < n) {
                const uint16_t s = scales[gn * groups + g];
                if (FMT == 0) {
                    const uint8_t* p = packed + gn * row_bytes + g * kTrit5GroupBytes;
                    const int j0 = part < 2 ? part * 7 : 14 + (part - 2) * 6;
                    const int j1 = part < 2 ? j0 + 7 : j0 + 6;
                    for (int j = j0; j < j1; ++j) {
                        uint32_t v = p[j];
                        const int cnt = j < 25 ? 5 : 3;
                        for (int i = 0; i < cnt; ++i) {
                            const uint32_t qd = v / 3u;
                            dst[5 * j + i] = code_times_scale(v - 3u * qd, s);
                            v = qd;
                        }
                    }
                } else {
                    const uint8_t* p = packed + gn * row_bytes + g * (kGroup / 4) + part * 8;
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t v = p[j];
                        for (int i = 0; i < 4; ++i)
                            dst[part * 32 + 4 * j + i] = code_times_scale((v >> (2 * i)) & 3u, s);
                    }
                }
            } else {
                for (int i = 0; i < 32; ++i) dst[part * 32 + i] = 0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            half8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = wm + i * 16 + (lane & 15);
                const int rb = wn + i * 16 + (lane & 15);
                const int kk = ks + 8 * (lane >> 4);
                a[i] = *reinterpret_cast<const half8*>(As + ra * kLdsStride + kk);
                b[i] = *reinterpret_cast<const half8*>(Bs + rb * kLdsStride + kk);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // lane holds D[4 * (lane / 16) + r][lane % 16] of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gm = m_base + wm + i * 16 + 4 * (lane >> 4) + r;
                const int64_t gn = n_base + wn + j * 16 + (lane & 15);
                if (gm < m && gn < n) {
                    const float v = acc[i][j][r];
                    if (y_f16)
                        reinterpret_cast<__half*>(y)[gm * n + gn] = __float2half_rn(v);
                    else
                        reinterpret_cast<float*>(y)[gm * n + gn] = v;
                }
            }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    const dim3 grid(unsigned(((n + BN - 1) / BN) * ((m + BM - 1) / BM)));
    if (fmt == 0)
        hipLaunchKernelGGL(gemm_simple_kernel<0>, grid, dim3(kThreads), 0, stream, packed, scales,
                           x, m, n, k, y, y_f16);
    else
        hipLaunchKernelGGL(gemm_simple_kernel<1>, grid, dim3(kThreads), 0, stream, packed, scales,
                           x, m, n, k, y, y_f16);
    return hipGetLastError();
}

}  // namespace tl
