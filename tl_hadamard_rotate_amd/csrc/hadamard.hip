// Signed block-Hadamard rotation of activations, 1024-wide blocks:
//   out_b = (1/32) H (s_b * x_b),  H the natural-order (Sylvester) Hadamard matrix.
// The transform is the orthogonal block rotation that was folded into the
// weights; the activations must receive it at run time (page "A 27-billion
// model that fits in 8.6 GB", paragraphs 2 and 3; signs: page "OpenBonsai",
// section "How it works", step 1).
//
// Fast Walsh-Hadamard transform in fp32, one wave per pair of blocks:
//   layout A: lane q (0..31) of a half-wave holds element i = 256c + 8q + e for
//             c = 0..3, e = 0..7 (four coalesced 16-byte loads per lane);
//             butterflies on index bits 0-2 and 8-9 in registers.
//   LDS transpose to layout B: lane (c, e) holds i = 256c + 8r + e, r = 0..31;
//             butterflies on bits 3-7 in registers.
//   LDS transpose back to layout A, round to binary16, four 16-byte stores.
// LDS word address of element (c, q, e) is 296c + 9q + e: with 32 or 64 banks
// both the A-side (q varies) and the B-side ((c, e) varies) accesses of a
// half-wave hit distinct banks, and a half-wave stride of 1184 words (= 32 mod
// 64) keeps the two half-waves apart.  Every address is a lane base plus an
// immediate offset.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalfStride = 1184;   // words per half-wave block in LDS

__device__ __forceinline__ int lds_addr(int c, int q, int e) { return 296 * c + 9 * q + e; }

__global__ __launch_bounds__(kThreads) void hadamard_kernel(
    const uint16_t* x, const int8_t* __restrict__ signs, int64_t total_blocks,
    int64_t k_blocks, uint16_t* out) {   // x and out may be the same buffer
    __shared__ float lds[kWaves * 2 * kHalfStride];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int q = lane & 31;
    const int64_t blk = (int64_t(blockIdx.x) * kWaves + wave) * 2 + half;
    const bool active = blk < total_blocks;
    float* my = lds + (wave * 2 + half) * kHalfStride;

    float v[32];   // v[8c + e] is element 256c + 8q + e (layout A)
    if (active) {
        const uint16_t* src = x + blk * kBlock + 8 * q;
        const int8_t* sg = signs + (blk % k_blocks) * kBlock + 8 * q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 raw = *reinterpret_cast<const uint4*>(src + 256 * c);
            const uint2 sraw = *reinterpret_cast<const uint2*>(sg + 256 * c);
            const __half* h = reinterpret_cast<const __half*>(&raw);
            const int8_t* s = reinterpret_cast<const int8_t*>(&sraw);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // 1/32 is folded in here: exact in fp32, so it commutes with the sums
                const float f = __half2float(h[e]);
                v[8 * c + e] = s[e] < 0 ? -0.03125f * f : 0.03125f * f;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
    }

    // layout A: butterflies over e bits (0, 1, 2) and c bits (index bits 8, 9)
#pragma unroll
    for (int hb = 1; hb < 8; hb <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (!(e & hb)) {
                    const float a = v[8 * c + e], b = v[8 * c + e + hb];
                    v[8 * c + e] = a + b;
                    v[8 * c + e + hb] = a - b;
                }
    }
#pragma unroll
    for (int hc = 1; hc < 4; hc <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (!(c & hc))
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = v[8 * c + e], b = v[8 * (c + hc) + e];
                    v[8 * c + e] = a + b;
                    v[8 * (c + hc) + e] = a - b;
                }
    }

#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) my[lds_addr(c, q, e)] = v[8 * c + e];
    __syncthreads();

    // layout B: this lane is (cb, eb); w[r] is element 256 cb + 8 r + eb
    const int cb = q >> 3, eb = q & 7;
    float w[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) w[r] = my[lds_addr(cb, r, eb)];
#pragma unroll
    for (int hr = 1; hr < 32; hr <<= 1) {
#pragma unroll
        for (int r = 0; r < 32; ++r)
            if (!(r & hr)) {
                const float a = w[r], b = w[r + hr];
                w[r] = a + b;
                w[r + hr] = a - b;
            }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 32; ++r) my[lds_addr(cb, r, eb)] = w[r];
    __syncthreads();

    if (active) {
        uint16_t* dst = out + blk * kBlock + 8 * q;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint4 raw;
            __half* h = reinterpret_cast<__half*>(&raw);
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = __float2half_rn(my[lds_addr(c, q, e)]);
            *reinterpret_cast<uint4*>(dst + 256 * c) = raw;
        }
    }
}

}  // namespace

hipError_t launch_hadamard(const uint16_t* x, const int8_t* signs, int64_t m, int64_t k,
                           uint16_t* out, hipStream_t stream) {
    const int64_t k_blocks = k / kBlock;
    const int64_t total = m * k_blocks;
    const int64_t per_wg = 2 * kWaves;
    const int64_t grid = (total + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(hadamard_kernel, dim3(unsigned(grid)), dim3(kThreads), 0, stream, x, signs,
                       total, k_blocks, out);
    return hipGetLastError();
}

}  // namespace tl
