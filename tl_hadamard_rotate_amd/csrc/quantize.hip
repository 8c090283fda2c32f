// Weight-side quantiser: rotate real-valued weight rows with the activations'
// signed 1024-block Hadamard transform (folded into the weights: page
// "OpenBonsai", section "How it works", step 1; page "A 27-billion model that
// fits in 8.6 GB", paragraph 2), then round each row to ternary g128 (step 2
// of the same section, there by GPTQ on calibration data; here round to
// nearest with the group's mean |w'| as its binary16 scale).
//
//   w'[1024 b + i] = (1/32) sum_j H[i, j] s[1024 b + j] w[1024 b + j]
//   S = binary16(mean of |w'| over a group of 128), c = rint(w' / S) clipped
//   to [-1, 1] (ties to even: |w'| = S / 2 gives 0), c = 0 where S = 0.
//
// One workgroup of 256 threads per (row, 1024-block); thread t holds
// elements 4t..4t+3.  The butterflies run in fp32 in a fixed order (index
// bits 0-1 in registers, bits 2-9 through two alternating LDS buffers, one
// barrier per stage), so results are bitwise reproducible.  Offline work, once
// per weight.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kThreads = 256;

constexpr int kUnits = 4;   // (row, 1024-block) units per workgroup, loaded together

// One unit: elements 4t..4t+3 of row `row`, block `blk`, already loaded.
__device__ __forceinline__ void quantize_unit(const float4 wv, const char4 sv, int64_t row,
                                              int64_t blk, int64_t k, int t,
                                              float (&buf)[2][kBlock], int8_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales) {
    const int64_t base = row * k + blk * kBlock + 4 * t;
    float v[4] = {sv.x < 0 ? -wv.x : wv.x, sv.y < 0 ? -wv.y : wv.y, sv.z < 0 ? -wv.z : wv.z,
                  sv.w < 0 ? -wv.w : wv.w};
    // index bits 0 and 1: (a, b) -> (a + b, a - b)
    float a0 = v[0] + v[1], a1 = v[0] - v[1], a2 = v[2] + v[3], a3 = v[2] - v[3];
    v[0] = a0 + a2;
    v[1] = a1 + a3;
    v[2] = a0 - a2;
    v[3] = a1 - a3;
    // index bits 2..9 (thread bits 0..7) through LDS, one barrier per stage
#pragma unroll
    for (int bit = 2; bit < 10; ++bit) {
        float* b = buf[bit & 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) b[4 * t + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * t + e;
            const float p = b[i ^ (1 << bit)];
            v[e] = (i >> bit) & 1 ? p - v[e] : v[e] + p;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] *= 1.0f / 32.0f;
        s += __builtin_fabsf(v[e]);
    }
    // group of 128 = the 32 threads 32g .. 32g + 31 (half a wave)
    s += __shfl_xor(s, 16, 32);
    s += __shfl_xor(s, 8, 32);
    s += __shfl_xor(s, 4, 32);
    s += __shfl_xor(s, 2, 32);
    s += __shfl_xor(s, 1, 32);
    const __half sh = __float2half_rn(s * (1.0f / 128.0f));
    const float sc = __half2float(sh);
    const float half_s = 0.5f * sc;
    int8_t c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        c[e] = sc != 0.0f && __builtin_fabsf(v[e]) > half_s ? (v[e] > 0.0f ? 1 : -1) : 0;
    *reinterpret_cast<char4*>(codes + base) = char4{c[0], c[1], c[2], c[3]};
    if ((t & 31) == 0)
        scales[row * (k / kGroup) + blk * (kBlock / kGroup) + (t >> 5)] = __half_as_ushort(sh);
}

// The loads of all units go out first, so a workgroup keeps kUnits x 4 KB
// in flight; the units are then rotated and rounded one after another.
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float* __restrict__ w,
                                                            const int8_t* __restrict__ signs,
                                                            int64_t k, int64_t units,
                                                            int8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ scales) {
    // two buffers, used by alternate stages: a stage's barrier also tells every
    // thread that the reads of the stage before the previous one are done
    __shared__ float buf[2][kBlock];
    const int t = threadIdx.x;
    const int64_t blocks = k / kBlock;
    // (row, block) of each unit: one division, then steps along the rows
    const int64_t u0 = int64_t(blockIdx.x) * kUnits;   // workgroup-uniform
    int64_t rows[kUnits], blks[kUnits];
    {
        int64_t r = u0 / blocks, b = u0 - r * blocks;
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            rows[j] = r;
            blks[j] = b;
            if (++b == blocks) {
                b = 0;
                ++r;
            }
        }
    }
    float4 wv[kUnits];
    char4 sv[kUnits];
#pragma unroll
    for (int j = 0; j < kUnits; ++j)
        if (u0 + j < units) {
            wv[j] = *reinterpret_cast<const float4*>(w + rows[j] * k + blks[j] * kBlock + 4 * t);
            sv[j] = *reinterpret_cast<const char4*>(signs + blks[j] * kBlock + 4 * t);
        }
#pragma unroll
    for (int j = 0; j < kUnits; ++j)
        if (u0 + j < units) quantize_unit(wv[j], sv[j], rows[j], blks[j], k, t, buf, codes, scales);
}

}  // namespace

hipError_t launch_quantize(const float* w, const int8_t* signs, int64_t n, int64_t k,
                           int8_t* codes, uint16_t* scales, hipStream_t stream) {
    const int64_t units = n * (k / kBlock);
    const int64_t grid = (units + kUnits - 1) / kUnits;
    hipLaunchKernelGGL(quantize_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, w,
                       signs, k, units, codes, scales);
    return hipGetLastError();
}

}  // namespace tl
