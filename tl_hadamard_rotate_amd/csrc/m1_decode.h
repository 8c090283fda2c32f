// Device building blocks of the M = 1 decode kernels for the 2-bit-slot
// packing (the single-linear kernel in gemv_m1.hip and the chain kernel in
// chain.hip): the per-lane activation images, the subnormal-class digit
// decode and the matrix-core diagonal products.  How they fit together is
// described at the top of gemv_m1.hip.
#pragma once

#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace m1 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = 4 * kWaves;          // 16-lane slots per workgroup
constexpr int kImgLane = 144;               // bytes per lane image (128 used; bank spread)
constexpr int kImgBlock = 16 * kImgLane;    // per 1024-block
constexpr int kRecBytes = 16;               // per (block, column): {2^(10+E), -sum_X, -sum_Y, 0}
constexpr int kMaxSegsPerChunk = 2048;      // LDS partial sums of one row chunk: 32 KB
constexpr size_t kLdsLimit = 160 * 1024;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;      // offset past every buffer range: loads return 0

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(uintptr_t((const __attribute__((address_space(3))) void*)(p)));
}

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// binary16 -> fp32 of bits h, and fp32 -> binary16 bits (round to nearest even)
__device__ __forceinline__ float h2f(uint32_t h) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}
__device__ __forceinline__ uint32_t f2h(float f) {
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}
__device__ __forceinline__ float pow2f(int e) {   // 2^e for -126 <= e <= 127
    return __builtin_bit_cast(float, uint32_t(127 + e) << 23);
}

// k offset (in the 1024-block) of the first of the 16 digits of e-word e of
// lane rank u, after the permlane32 exchange: e-words 0 and 2 belong to the
// column's first group, 1 and 3 to its second
__device__ __forceinline__ int eword_k(int u, int e) {
    const int q = u & 3;
    if (q < 2) return 64 * (u + ((e & 1) ? 2 : 0)) + ((e & 2) ? 32 : 0);
    return 64 * (u - ((e & 1) ? 0 : 2)) + 16 + ((e & 2) ? 32 : 0);
}

// Activation images.  Thread t works on block b = t / 32, column c = (t / 8)
// % 4, e-words ep and ep + 2 (ep = (t / 4) % 2: the column's first group for
// ep = 0, its second for ep = 1) of lane rank u = 4c + t % 4; the eight threads
// of a column are consecutive lanes, the four of a group a lane quad.  load_x
// issues the 4 loads of a thread, build_pass turns them into LDS images and,
// for the column, the record {2^(10+E), -sum_first x 2^(-10-E),
// -sum_second x 2^(-10-E)}.  One pass covers kThreads / 32 blocks.
__device__ __forceinline__ int img_u(int t) { return 4 * ((t >> 3) & 3) + (t & 3); }
__device__ __forceinline__ int img_ep(int t) { return (t >> 2) & 1; }

// cross-lane moves inside a lane quad / between the two quads of 8 lanes
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within 8
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(uint32_t, v)));
}

__device__ __forceinline__ void load_x(const uint16_t* x, int nb, int t, uint4 (&raw)[4]) {
    const int b = t >> 5;
    const int u = img_u(t);
    const int ep = img_ep(t);
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, nb * 2048, kRsrcWord3);
    // lanes past the last block issue nothing (loads that return zeros still
    // take the address units' time ahead of the weight loads); their raw is
    // left unset and never used
    if (t < nb * 32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t o = uint32_t((1024 * b + eword_k(u, ep + 2 * h)) * 2);
            raw[2 * h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, o, 0, 0));
            raw[2 * h + 1] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, o + 16, 0, 0));
        }
    }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// s + (low or high binary16 half of w), in fp32 with one rounding (the half
// converts exactly): one mixed-precision fma instead of a conversion and an add
__device__ __forceinline__ float add_lo_half(float s, uint32_t w) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(s) : "v"(w));
    return s;
}
__device__ __forceinline__ float add_hi_half(float s, uint32_t w) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(s) : "v"(w));
    return s;
}
__device__ __forceinline__ _Float16 pow2h(int e) {   // 2^e for -14 <= e <= 15
    return __builtin_bit_cast(_Float16, uint16_t((15 + e) << 10));
}

// SUMS: also the record's group sums (a kernel that takes them from the
// matrix cores passes false; its records hold {2^(10+E), 0, 0, 0}).
template <bool SUMS = true>
__device__ inline void build_pass(const uint4 (&raw)[4], int nb, int t, uint8_t* img, uint8_t* rec) {
    const bool live = t < nb * 32;
    const int b = live ? t >> 5 : 0;
    const int u = img_u(t);
    const int ep = img_ep(t);
    // largest |x| of the column (bit patterns of non-negative binary16 values
    // order like the values): packed 16-bit maxima of the magnitudes
    u16x2 mv = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            mv = __builtin_elementwise_max(mv, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    }
    uint32_t m = max(uint32_t(mv.x), uint32_t(mv.y));
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    m = max(m, dpp<kDppHalfMirror>(m));
    int ex = 0;
    if (m >= 0x400u)
        ex = int(m >> 10) - 15;
    else if (m != 0u)
        ex = (31 - __builtin_clz(m)) - 24;
    // At least -5, so that the three pre-scales below are binary16 numbers.
    // Nothing is lost: a column whose largest |x| is below 2^-5 is scaled by
    // 2^15 (instead of more) and every binary16 x times 2^11..2^15 is still
    // an exact normal binary16 number; the sums scale by a power of two.
    ex = max(ex, -5);
    // pre-scale of in-word position j (its digit decodes to d * 2^(s_j - 24)),
    // s_j = 4, 6, 4, 6, 8, 4, 6, 8: factor 2^(14 - s_j - ex)
    const _Float16 f4 = pow2h(10 - ex), f6 = pow2h(8 - ex), f8 = pow2h(6 - ex);
    const _Float16 fc[8] = {f4, f6, f4, f6, f8, f4, f6, f8};
    u32x4* dst = reinterpret_cast<u32x4*>(img + b * kImgBlock + u * kImgLane);
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // x[16 h' + i] (i = 0..15 of this e-word pair) at half i of w
        const uint32_t w[8] = {raw[2 * h].x, raw[2 * h].y, raw[2 * h].z, raw[2 * h].w,
                               raw[2 * h + 1].x, raw[2 * h + 1].y, raw[2 * h + 1].z,
                               raw[2 * h + 1].w};
        if constexpr (SUMS) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sum = add_hi_half(add_lo_half(sum, w[j]), w[j]);
        }
        // pair j faces digits (j, 8 + j): halves j and 8 + j side by side,
        // times the pair's factor (binary16 product, rounded once as the
        // fp32 product rounded to binary16 would be)
        uint32_t out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t pr = __builtin_amdgcn_perm(w[4 + j / 2], w[j / 2],
                                                      (j & 1) ? 0x07060302u : 0x05040100u);
            out[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, pr) * half2v{fc[j], fc[j]});
        }
        const int e = ep + 2 * h;
        if (live) {
            dst[2 * e] = u32x4{out[0], out[1], out[2], out[3]};
            dst[2 * e + 1] = u32x4{out[4], out[5], out[6], out[7]};
        }
    }
    // the column's group sums: over the lane quad, then the other group's
    // from the other quad
    float other = 0.0f;
    if constexpr (SUMS) {
        sum += dppf<kDppXor1>(sum);
        sum += dppf<kDppXor2>(sum);
        other = dppf<kDppHalfMirror>(sum);
    }
    if (live && (t & 7) == 0) {
        const float unit = pow2f(-10 - ex);
        *reinterpret_cast<float4*>(rec + (b * 4 + (u >> 2)) * kRecBytes) =
            float4{pow2f(10 + ex), -sum * unit, -other * unit, 0.0f};
    }
}

// load_x from the rotated activations in LDS
__device__ __forceinline__ void load_x_lds(const uint16_t* xrot, int nb, int t, uint4 (&raw)[4]) {
    const int b = t >> 5;
    const int u = img_u(t);
    const int ep = img_ep(t);
    if (t < nb * 32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4* src = reinterpret_cast<const uint4*>(xrot + 1024 * b + eword_k(u, ep + 2 * h));
            raw[2 * h] = src[0];
            raw[2 * h + 1] = src[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = uint4{0, 0, 0, 0};
    }
}

__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(half8, u32x4{a, b, c, d});
}

// one e-word into D: two MFMAs over its 16 digits
__device__ __forceinline__ float4v mac_eword(uint32_t e, const half8& a_lo, const half8& a_hi,
                                             float4v acc) {
    const uint32_t l4 = e << 4, r6 = e >> 6;
    const half8 b_lo = as_h8(l4 & 0x00300030u, l4 & 0x00C000C0u, e & 0x00300030u, e & 0x00C000C0u);
    const half8 b_hi = as_h8(e & 0x03000300u, r6 & 0x00300030u, r6 & 0x00C000C0u, r6 & 0x03000300u);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, b_lo, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, b_hi, acc, 0, 0, 0);
}

// 16 bits of 1-bit codes (bits 16h .. 16h + 15 of w) as the 2-bit-slot word of
// the same 16 weights: bit i moves to bit 2i + 1 (digit 2b)
__device__ __forceinline__ uint32_t spread_bits(uint32_t w, int h) {
    uint32_t v = __builtin_amdgcn_perm(0u, w, h ? 0x0C030C02u : 0x0C010C00u);   // byte per 16 bits
    v = (v | (v << 4)) & 0x0F0F0F0Fu;
    v = (v | (v << 2)) & 0x33333333u;
    v = (v | (v << 1)) & 0x55555555u;
    return v << 1;
}

__device__ __forceinline__ float pick(const float4v& d, int r) {
    return r == 0 ? d[0] : (r == 1 ? d[1] : (r == 2 ? d[2] : d[3]));
}

}  // namespace m1
}  // namespace tl
