// Packing of ternary codes into the two byte formats, and the reverse.
// Formats: 5 trits per byte in base 3 (26 bytes per 128-group) and one 2-bit
// slot per weight; both hold digit d = code + 1.  The two packings carry the
// same weights and differ only in layout (page "A 27-billion model that fits
// in 8.6 GB", paragraph 5).  The 1-bit format holds codes -1 and +1 as one bit
// b = (code + 1) / 2 each, eight to a byte, first weight in the least
// significant bit (page "How Prism ML Squeezed a 27B Model Into 3.9 GB", list
// "Two formats ship today").  Bit-exact integer work; offline, once per weight.
#include "tl_internal.h"

namespace tl {
namespace {

constexpr int kThreads = 256;

// digit of one code; codes outside {-1,0,1} become digit 1 (code 0) and are counted
__device__ __forceinline__ uint32_t code_digit(int8_t c, uint32_t& bad) {
    uint32_t ok = (c >= -1) & (c <= 1);
    bad += ok ^ 1u;
    return ok ? uint32_t(c + 1) : 1u;
}

// One thread per output byte of a 26-byte group: byte j < 25 takes codes
// 5j..5j+4, byte 25 takes codes 125..127 and two pad digits of 1.
__global__ __launch_bounds__(kThreads) void pack_trit5_kernel(
    const int8_t* __restrict__ codes, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int32_t* __restrict__ bad_count) {
    const int64_t row_bytes = (k / kGroup) * kTrit5GroupBytes;
    const int64_t total = n * row_bytes;
    uint32_t bad = 0;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const int64_t row = idx / row_bytes;
        const int64_t rb = idx - row * row_bytes;
        const int64_t g = rb / kTrit5GroupBytes;
        const int j = int(rb - g * kTrit5GroupBytes);
        const int8_t* src = codes + row * k + g * kGroup + 5 * j;
        const int cnt = j < 25 ? 5 : 3;
        uint32_t val = 0, w = 1;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint32_t d = i < cnt ? code_digit(src[i], bad) : 1u;
            val += d * w;
            w *= 3;
        }
        packed[idx] = uint8_t(val);
    }
    if (bad_count && bad) atomicAdd(bad_count, int32_t(bad));
}

// One thread per output dword of the 2-bit format (16 codes in, 4 bytes out).
__global__ __launch_bounds__(kThreads) void pack_slot2_kernel(
    const int8_t* __restrict__ codes, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int32_t* __restrict__ bad_count) {
    const int64_t total = n * k / 16;
    uint32_t bad = 0;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const int4 raw = reinterpret_cast<const int4*>(codes)[idx];
        const int8_t* c = reinterpret_cast<const int8_t*>(&raw);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) word |= code_digit(c[i], bad) << (2 * i);
        reinterpret_cast<uint32_t*>(packed)[idx] = word;
    }
    if (bad_count && bad) atomicAdd(bad_count, int32_t(bad));
}

// One thread per output dword of the 1-bit format (32 codes in, 4 bytes out);
// codes other than -1 and +1 become bit 1 (code +1) and are counted.
__global__ __launch_bounds__(kThreads) void pack_bit1_kernel(
    const int8_t* __restrict__ codes, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int32_t* __restrict__ bad_count) {
    const int64_t total = n * k / 32;
    uint32_t bad = 0;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const int4* src = reinterpret_cast<const int4*>(codes) + 2 * idx;
        uint32_t word = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int4 raw = src[half];
            const int8_t* c = reinterpret_cast<const int8_t*>(&raw);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                bad += (c[i] != -1) & (c[i] != 1);
                word |= uint32_t(c[i] != -1) << (16 * half + i);
            }
        }
        reinterpret_cast<uint32_t*>(packed)[idx] = word;
    }
    if (bad_count && bad) atomicAdd(bad_count, int32_t(bad));
}

__global__ __launch_bounds__(kThreads) void unpack_trit5_kernel(
    const uint8_t* __restrict__ packed, int64_t n, int64_t k, int8_t* __restrict__ codes) {
    const int64_t row_bytes = (k / kGroup) * kTrit5GroupBytes;
    const int64_t total = n * row_bytes;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const int64_t row = idx / row_bytes;
        const int64_t rb = idx - row * row_bytes;
        const int64_t g = rb / kTrit5GroupBytes;
        const int j = int(rb - g * kTrit5GroupBytes);
        int8_t* dst = codes + row * k + g * kGroup + 5 * j;
        uint32_t v = packed[idx];
        const int cnt = j < 25 ? 5 : 3;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const uint32_t q = v / 3u;
            const uint32_t d = v - 3u * q;
            v = q;
            if (i < cnt) dst[i] = int8_t(int(d > 2u ? 1u : d) - 1);
        }
    }
}

__global__ __launch_bounds__(kThreads) void unpack_slot2_kernel(
    const uint8_t* __restrict__ packed, int64_t n, int64_t k, int8_t* __restrict__ codes) {
    const int64_t total = n * k / 4;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const uint32_t b = packed[idx];
        uint32_t out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t d = (b >> (2 * i)) & 3u;
            d = d > 2u ? 1u : d;
            out |= (uint32_t(uint8_t(int8_t(int(d) - 1)))) << (8 * i);
        }
        reinterpret_cast<uint32_t*>(codes)[idx] = out;
    }
}

// One thread per input byte of the 1-bit format: 8 codes out.
__global__ __launch_bounds__(kThreads) void unpack_bit1_kernel(
    const uint8_t* __restrict__ packed, int64_t n, int64_t k, int8_t* __restrict__ codes) {
    const int64_t total = n * k / 8;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const uint32_t b = packed[idx];
        uint32_t out[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            out[i >> 2] |= ((b >> i) & 1u ? 0x01u : 0xFFu) << (8 * (i & 3));
        reinterpret_cast<uint2*>(codes)[idx] = uint2{out[0], out[1]};
    }
}

// One thread per input dword of the 1-bit format: its 32 bits b become the
// 2-bit digits 2b (code -1 -> digit 0, +1 -> digit 2), two output dwords.
__global__ __launch_bounds__(kThreads) void bit1_to_slot2_kernel(
    const uint8_t* __restrict__ bit1, int64_t total, uint8_t* __restrict__ slot2) {
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(bit1)[idx];
        uint32_t out[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // spread 16 bits to the even bit positions of a dword, then move them up one
            uint32_t v = (w >> (16 * h)) & 0xFFFFu;
            v = (v | (v << 8)) & 0x00FF00FFu;
            v = (v | (v << 4)) & 0x0F0F0F0Fu;
            v = (v | (v << 2)) & 0x33333333u;
            v = (v | (v << 1)) & 0x55555555u;
            out[h] = v << 1;
        }
        reinterpret_cast<uint2*>(slot2)[idx] = uint2{out[0], out[1]};
    }
}

// One thread per 128-code group: the dense trit packing rewritten as 2-bit
// slots (32 bytes per group).  Bytes above 242, which the packer never
// writes, decode as their base-3 digits, as in unpack_trit5_kernel.  The 26
// bytes are read as the 7 dwords from the one holding the group's first byte
// (in bounds for every group: the last group of a row starts at 2 mod 4).
template <int O>
__device__ __forceinline__ void trit5_group_to_slot2(const uint32_t (&dw)[7], uint32_t (&w)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0;
#pragma unroll
    for (int j = 0; j < 26; ++j) {
        uint32_t v = (dw[(O + j) >> 2] >> (8 * ((O + j) & 3))) & 0xFFu;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int c = 5 * j + i;
            const uint32_t q = (v * 171u) >> 9;   // v / 3 for v < 256
            if (c < kGroup) w[c >> 4] |= (v - 3u * q) << (2 * (c & 15));
            v = q;
        }
    }
}

__global__ __launch_bounds__(kThreads) void trit5_to_slot2_kernel(
    const uint8_t* __restrict__ trit5, int64_t n, int64_t k, uint8_t* __restrict__ slot2) {
    const int64_t groups = k / kGroup;
    const int64_t total = n * groups;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const int64_t row = idx / groups, g = idx - row * groups;
        const int64_t start = row * groups * kTrit5GroupBytes + g * kTrit5GroupBytes;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(trit5 + (start & ~int64_t(3)));
        uint32_t dw[7], w[8];
#pragma unroll
        for (int i = 0; i < 7; ++i) dw[i] = src[i];
        if (start & 3)
            trit5_group_to_slot2<2>(dw, w);
        else
            trit5_group_to_slot2<0>(dw, w);
        uint4* dst = reinterpret_cast<uint4*>(slot2 + row * (k / 4) + g * 32);
        dst[0] = uint4{w[0], w[1], w[2], w[3]};
        dst[1] = uint4{w[4], w[5], w[6], w[7]};
    }
}

unsigned grid_for(int64_t total) {
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    return unsigned(blocks);
}

// One thread per packed byte: counts the bytes that are not valid encodings
// (a 2-bit slot holding 3; a dense-trit byte above 242, or a group's last
// byte whose two pad digits are not 1, i.e. outside 108..134).
__global__ __launch_bounds__(kThreads) void count_invalid_kernel(
    const uint8_t* __restrict__ packed, int64_t total, int64_t group_bytes, int fmt,
    int32_t* __restrict__ count) {
    uint32_t bad = 0;
    for (int64_t idx = int64_t(blockIdx.x) * kThreads + threadIdx.x; idx < total;
         idx += int64_t(gridDim.x) * kThreads) {
        const uint32_t v = packed[idx];
        if (fmt == 0) {
            const bool last = idx % group_bytes == group_bytes - 1;
            bad += last ? (v < 108u || v > 134u) : (v > 242u);
        } else {
            bad += ((v & 0x55u) & ((v >> 1) & 0x55u)) != 0u;
        }
    }
    if (bad) atomicAdd(count, int32_t(bad));
}

}  // namespace

hipError_t launch_count_invalid(const uint8_t* packed, int64_t n, int64_t k, int fmt,
                                int32_t* count, hipStream_t stream) {
    if (fmt == 2) return hipSuccess;   // every byte of the 1-bit format is valid
    const int64_t total = fmt == 0 ? n * (k / kGroup) * kTrit5GroupBytes : n * k / 4;
    hipLaunchKernelGGL(count_invalid_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                       packed, total, int64_t(kTrit5GroupBytes), fmt, count);
    return hipGetLastError();
}

hipError_t launch_pack(const int8_t* codes, int64_t n, int64_t k, int fmt, uint8_t* packed,
                       int32_t* bad_count, hipStream_t stream) {
    if (fmt == 0) {
        const int64_t total = n * (k / kGroup) * kTrit5GroupBytes;
        hipLaunchKernelGGL(pack_trit5_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                           codes, n, k, packed, bad_count);
    } else if (fmt == 2) {
        hipLaunchKernelGGL(pack_bit1_kernel, dim3(grid_for(n * k / 32)), dim3(kThreads), 0, stream,
                           codes, n, k, packed, bad_count);
    } else {
        const int64_t total = n * k / 16;
        hipLaunchKernelGGL(pack_slot2_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                           codes, n, k, packed, bad_count);
    }
    return hipGetLastError();
}

hipError_t launch_trit5_to_slot2(const uint8_t* trit5, int64_t n, int64_t k, uint8_t* slot2,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(trit5_to_slot2_kernel, dim3(grid_for(n * (k / kGroup))), dim3(kThreads), 0,
                       stream, trit5, n, k, slot2);
    return hipGetLastError();
}

hipError_t launch_bit1_to_slot2(const uint8_t* bit1, int64_t n, int64_t k, uint8_t* slot2,
                               hipStream_t stream) {
    const int64_t total = n * k / 32;
    hipLaunchKernelGGL(bit1_to_slot2_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                       bit1, total, slot2);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int fmt, int8_t* codes,
                         hipStream_t stream) {
    if (fmt == 0) {
        const int64_t total = n * (k / kGroup) * kTrit5GroupBytes;
        hipLaunchKernelGGL(unpack_trit5_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                           packed, n, k, codes);
    } else if (fmt == 2) {
        hipLaunchKernelGGL(unpack_bit1_kernel, dim3(grid_for(n * k / 8)), dim3(kThreads), 0,
                           stream, packed, n, k, codes);
    } else {
        const int64_t total = n * k / 4;
        hipLaunchKernelGGL(unpack_slot2_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                           packed, n, k, codes);
    }
    return hipGetLastError();
}

}  // namespace tl
