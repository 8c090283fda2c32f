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
// One wave per (row, 1024-block) unit, lane l holding elements 16l .. 16l + 15:
// index bits 0-3 are butterflied in registers and bits 4-9 (the lane bits)
// with cross-lane exchanges, so no LDS storage and no workgroup barrier are
// needed; each wave loads its two units before working on either.  The
// exchanges are split between the VALU (DPP quad permutes for lane bits 0-1, a
// swap of the wave's halves for bit 5) and the LDS unit's lane permute (bits
// 2-4): all of them through the permute was bound by it, all of them on the
// VALU by the VALU.
// fp32 throughout in a fixed order, so results are bitwise reproducible.
// Offline work, once per weight.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaveUnits = 2;   // (row, 1024-block) units per wave, loaded together

// v of lane l ^ m: DPP quad permutes for m = 1, 2, a swap of the wave's
// halves for m = 32, a lane permute otherwise
__device__ __forceinline__ float lane_xor(float v, int m, int l) {
    const int b = __builtin_bit_cast(int, v);
    if (m == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false));
    if (m == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false));
    if (m == 32) {
        const auto sw = __builtin_amdgcn_permlane32_swap(uint32_t(b), uint32_t(b), false, false);
        return __builtin_bit_cast(float, l < 32 ? sw[1] : sw[0]);
    }
    return __shfl_xor(v, m, 64);
}

// One wave, one unit: lane l holds elements 16l .. 16l + 15 of the block.
// Index bits 0-3 are butterflied in registers, bits 4-9 (lane bits 0-5)
// across lanes; fp32 throughout in a fixed order.
__device__ __forceinline__ void quantize_wave_unit(const float4 (&wv)[4], const uint4 sv,
                                                   int64_t row, int64_t blk, int64_t k, int l,
                                                   int8_t* __restrict__ codes,
                                                   uint16_t* __restrict__ scales) {
    float v[16];
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float f[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * i + e;
            const bool neg = (sw[j >> 2] >> (8 * (j & 3) + 7)) & 1u;
            v[j] = neg ? -f[e] : f[e];
        }
    }
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (!(j & h)) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        // partner values first (16 exchanges in flight), then p + sign * v:
        // v + p in the lower lane of a pair, p - v in the upper (exact sign)
        const float sgn = (l & m) ? -1.0f : 1.0f;
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = lane_xor(v[j], m, l);
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = __builtin_fmaf(v[j], sgn, p[j]);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        v[j] *= 1.0f / 32.0f;
        s += __builtin_fabsf(v[j]);
    }
    // group of 128 = the 8 lanes 8g .. 8g + 7
    s += __shfl_xor(s, 4, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 1, 64);
    const __half sh = __float2half_rn(s * (1.0f / 128.0f));
    const float sc = __half2float(sh);
    const float half_s = 0.5f * sc;
    uint32_t cw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int c = sc != 0.0f && __builtin_fabsf(v[j]) > half_s ? (v[j] > 0.0f ? 1 : -1) : 0;
        cw[j >> 2] |= (uint32_t(c) & 0xFFu) << (8 * (j & 3));
    }
    *reinterpret_cast<uint4*>(codes + row * k + blk * kBlock + 16 * l) = uint4{cw[0], cw[1], cw[2], cw[3]};
    if ((l & 7) == 0)
        scales[row * (k / kGroup) + blk * (kBlock / kGroup) + (l >> 3)] = __half_as_ushort(sh);
}

// Each wave handles kWaveUnits consecutive units, all of whose loads go out
// first; no LDS and no workgroup barrier.
__global__ __launch_bounds__(kThreads) void quantize_kernel(const float* __restrict__ w,
                                                            const int8_t* __restrict__ signs,
                                                            int64_t k, int64_t units,
                                                            int8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ scales) {
    const int l = threadIdx.x & 63;
    const int64_t blocks = k / kBlock;
    const int64_t u0 = (int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6)) * kWaveUnits;
    int64_t rows[kWaveUnits], blks[kWaveUnits];
    {
        int64_t r = u0 / blocks, b = u0 - r * blocks;
#pragma unroll
        for (int j = 0; j < kWaveUnits; ++j) {
            rows[j] = r;
            blks[j] = b;
            if (++b == blocks) {
                b = 0;
                ++r;
            }
        }
    }
    float4 wv[kWaveUnits][4];
    uint4 sv[kWaveUnits];
#pragma unroll
    for (int j = 0; j < kWaveUnits; ++j)
        if (u0 + j < units) {
            const float4* src = reinterpret_cast<const float4*>(w + rows[j] * k + blks[j] * kBlock + 16 * l);
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[j][i] = src[i];
            sv[j] = *reinterpret_cast<const uint4*>(signs + blks[j] * kBlock + 16 * l);
        }
#pragma unroll
    for (int j = 0; j < kWaveUnits; ++j)
        if (u0 + j < units) quantize_wave_unit(wv[j], sv[j], rows[j], blks[j], k, l, codes, scales);
}

}  // namespace

hipError_t launch_quantize(const float* w, const int8_t* signs, int64_t n, int64_t k,
                           int8_t* codes, uint16_t* scales, hipStream_t stream) {
    const int64_t units = n * (k / kBlock);
    const int64_t per_wg = int64_t(kThreads / 64) * kWaveUnits;
    const int64_t grid = (units + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(quantize_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, w,
                       signs, k, units, codes, scales);
    return hipGetLastError();
}

}  // namespace tl
