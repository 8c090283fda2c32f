// Prefill products for every packing, and the layout of their workspace.
// The matrix-core kernels read 2-bit slots; the dense trit and 1-bit packings
// are rewritten as 2-bit slots once per call (one pass over the weights, small
// next to the product: prompt processing is compute-bound, so the denser
// format only has to be read once) into the start of the caller's workspace.
// The fp16 product's K-split partial sums follow at the next 256-byte
// boundary.
//
// bfloat16 activations take the same binary16 product.  A bfloat16 number has
// 8 significant bits, a binary16 number 11, so a bfloat16 row scaled by a
// power of two 2^-e that brings its largest |x| into [2^14, 2^15) converts to
// binary16 exactly (every element down to 2^-17 of that range; smaller ones
// round, at most 2^-25 of the row's largest |x|).  The product of the scaled
// row is the true product times 2^-e, exactly up to its fp32 sums, and the
// epilogue multiplies the outputs by 2^e.  Workspace after the rewrite: the
// binary16 copy [M, K], then the row factors 2^e (fp32 [M]), then the K-split
// partial sums.
#include "tl_internal.h"

namespace tl {
namespace {

int64_t rewrite_bytes(int64_t n, int64_t k, int fmt) {
    return fmt == 1 ? 0 : ((n * (k / 4) + 255) / 256) * 256;
}

// the 2-bit-slot weights the kernels read: the packed codes themselves, or
// their rewrite into the workspace
hipError_t slot2_weights(const uint8_t* packed, int fmt, int64_t n, int64_t k, void* ws,
                         const uint8_t** out, hipStream_t stream) {
    if (fmt == 1) {
        *out = packed;
        return hipSuccess;
    }
    uint8_t* s2 = static_cast<uint8_t*>(ws);
    const hipError_t e = fmt == 0 ? launch_trit5_to_slot2(packed, n, k, s2, stream)
                                  : launch_bit1_to_slot2(packed, n, k, s2, stream);
    *out = s2;
    return e;
}

constexpr int kCvtThreads = 256;
constexpr int kCvtRegs = 9;   // 16-byte pieces a thread keeps: rows up to 9 * 256 * 8 = 18432

int64_t align256(int64_t b) { return ((b + 255) / 256) * 256; }

__device__ __forceinline__ uint32_t bf16_pair_max(uint32_t w) {
    const uint32_t a = w & 0x7FFF7FFFu;   // magnitudes order like their bit patterns
    return max(a & 0xFFFFu, a >> 16);
}

__device__ __forceinline__ uint4 bf16_to_f16x8(uint4 v, float down) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_bit_cast(float, w[i] << 16) * down;
        const float hi = __builtin_bit_cast(float, w[i] & 0xFFFF0000u) * down;
        o[i] = uint32_t(__builtin_bit_cast(uint16_t, _Float16(lo))) |
               (uint32_t(__builtin_bit_cast(uint16_t, _Float16(hi))) << 16);
    }
    return uint4{o[0], o[1], o[2], o[3]};
}

// One workgroup per row: the row's largest magnitude, its exponent E, e = E -
// 14 (clamped to [-110, 113]: fp32 factors); then every element times 2^-e,
// rounded to binary16 (exact, see above).  fac[row] = 2^e.  Rows of up to
// kCvtRegs * kCvtThreads pieces are read once (kept in registers); longer
// rows are read twice.
__global__ __launch_bounds__(kCvtThreads) void bf16_rows_to_f16(const uint16_t* __restrict__ x,
                                                                int64_t k, uint16_t* __restrict__ out,
                                                                float* __restrict__ fac) {
    __shared__ uint32_t wmax[kCvtThreads / 64];
    const int64_t row = blockIdx.x;
    const uint4* src = reinterpret_cast<const uint4*>(x + row * k);
    uint4* dst = reinterpret_cast<uint4*>(out + row * k);
    const int chunks = int(k / 8);
    const int tid = threadIdx.x;
    const bool held = chunks <= kCvtRegs * kCvtThreads;
    uint4 v[kCvtRegs];
    uint32_t m = 0;
    if (held) {
#pragma unroll
        for (int i = 0; i < kCvtRegs; ++i) {
            const int c = tid + i * kCvtThreads;
            v[i] = c < chunks ? src[c] : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < kCvtRegs; ++i)
            m = max(m, max(max(bf16_pair_max(v[i].x), bf16_pair_max(v[i].y)),
                           max(bf16_pair_max(v[i].z), bf16_pair_max(v[i].w))));
    } else {
        for (int c = tid; c < chunks; c += kCvtThreads) {
            const uint4 u = src[c];
            m = max(m, max(max(bf16_pair_max(u.x), bf16_pair_max(u.y)),
                           max(bf16_pair_max(u.z), bf16_pair_max(u.w))));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), o)));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int i = 0; i < kCvtThreads / 64; ++i) m = max(m, wmax[i]);
    int ex = 0;
    if (m >= 0x80u)
        ex = int(m >> 7) - 127;
    else if (m != 0u)
        ex = (31 - __builtin_clz(m)) - 133;
    int e = ex - 14;
    e = e < -110 ? -110 : (e > 113 ? 113 : e);
    const float down = __builtin_bit_cast(float, uint32_t(127 - e) << 23);
    if (tid == 0) fac[row] = __builtin_bit_cast(float, uint32_t(127 + e) << 23);
    if (held) {
#pragma unroll
        for (int i = 0; i < kCvtRegs; ++i) {
            const int c = tid + i * kCvtThreads;
            if (c < chunks) dst[c] = bf16_to_f16x8(v[i], down);
        }
    } else {
        for (int c = tid; c < chunks; c += kCvtThreads) dst[c] = bf16_to_f16x8(src[c], down);
    }
}

}  // namespace

bool gemm_fits(int64_t m, int64_t n, int64_t k) { return gemm_slot2_fits(m, n, k); }

int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int fmt, bool bf16) {
    return rewrite_bytes(n, k, fmt) + (bf16 ? align256(m * k * 2) + align256(m * 4) : 0) +
           gemm_slot2_workspace_bytes(m, n, k);
}

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, void* ws,
                       int64_t ws_bytes, hipStream_t stream) {
    if (!gemm_fits(m, n, k) || ws_bytes < gemm_workspace_bytes(m, n, k, fmt, false))
        return hipErrorInvalidValue;
    const uint8_t* s2 = nullptr;
    const hipError_t e = slot2_weights(packed, fmt, n, k, ws, &s2, stream);
    if (e != hipSuccess) return e;
    const int64_t off = rewrite_bytes(n, k, fmt);
    void* part = ws ? static_cast<uint8_t*>(ws) + off : nullptr;
    return launch_gemm_slot2(s2, scales, x, m, n, k, y, y_f16, part, ws_bytes - off, stream);
}

hipError_t launch_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int fmt,
                            const uint16_t* x, int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            void* ws, int64_t ws_bytes, hipStream_t stream) {
    if (!gemm_fits(m, n, k) || ws_bytes < gemm_workspace_bytes(m, n, k, fmt, true))
        return hipErrorInvalidValue;
    const uint8_t* s2 = nullptr;
    hipError_t e = slot2_weights(packed, fmt, n, k, ws, &s2, stream);
    if (e != hipSuccess) return e;
    uint8_t* base = static_cast<uint8_t*>(ws) + rewrite_bytes(n, k, fmt);
    uint16_t* x16 = reinterpret_cast<uint16_t*>(base);
    float* fac = reinterpret_cast<float*>(base + align256(m * k * 2));
    uint8_t* part = base + align256(m * k * 2) + align256(m * 4);
    const int64_t left = ws_bytes - (part - static_cast<uint8_t*>(ws));
    hipLaunchKernelGGL(bf16_rows_to_f16, dim3(unsigned(m)), dim3(kCvtThreads), 0, stream, x, k, x16,
                       fac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_gemm_slot2(s2, scales, x16, m, n, k, y, y_f16, part, left, stream, fac);
}

}  // namespace tl
