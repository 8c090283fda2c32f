// Signed 1024-block Hadamard rotation of one activation row into LDS, for
// the GEMV kernels that rotate in their prologue (tl_linear at M = 1 and the
// decode chains):
//
//   x'[1024 b + i] = (1/32) sum_j H[i, j] s[1024 b + j] x[1024 b + j]
//
// (page "OpenBonsai", section "How it works", step 1; page "A 27-billion
// model that fits in 8.6 GB", paragraphs 2 and 3: the rotation folded into
// the weights has to be applied to the activations at run time.)
//
// One wave per block, the first half on the matrix cores.  With e = 32 a + b
// (a, b < 32), H_1024[e', e] = H_32[a', a] H_32[b', b] (the Sylvester matrix
// is the Kronecker power of H_2), so the block is the 32 x 32 matrix
// X[a][b] = s_e x_e and its transform is H_32 X H_32:
//  - stage 1, D = X H_32, is two v_mfma_f32_32x32x16_f16 (X in binary16 and
//    the +-1 entries are exact, the sums fp32): lane l feeds row a = l % 32 of
//    X (elements 16 kk + 8 (l / 32) + 0..7 of it for the kk-th MFMA) and the
//    same positions of column l % 32 of H_32;
//  - stage 2, H_32 D, runs as fp32 butterflies on the 16 accumulators of a
//    lane, which hold D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32], r = 0..15:
//    index bits 0, 1, 3, 4 of a are bits of r (in registers), bit 2 is the
//    lane half (one v_permlane32_swap per two registers).
// Each output is (1/32) times its exact value up to the fp32 roundings of a
// 32-term sum on the matrix cores and of 5 butterfly levels, rounded once to
// binary16 (tl_hadamard_rotate's butterfly tree rounds differently, so the two
// agree to within those bounds rather than bit for bit).
#pragma once

#include "tl_internal.h"

namespace tl {
namespace rot {

constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ uint32_t f2h(float f) {
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// one block's activations and signs for this lane: x[kk] holds elements
// 32 (l % 32) + 16 kk + 8 (l / 32) + 0..7 of the block, s[kk] their signs
struct In {
    uint4 x[2];
    u32x2v s[2];
};

// the loads of block blk (wave-uniform; nothing for blk >= nb); aux is the
// cache policy of the activation loads
template <int AUX = 0>
__device__ __forceinline__ void load(const uint16_t* x, const int8_t* signs, int nb, int blk, int lane,
                                     In& in) {
    const __amdgpu_buffer_rsrc_t xs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, nb * 2048, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ss =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, nb * 1024, kRsrcWord3);
    if (blk >= nb) return;
    const uint32_t e = uint32_t(1024 * blk + 32 * (lane & 31) + 8 * (lane >> 5));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        in.x[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, 2 * (e + 16 * kk), 0, AUX));
        in.s[kk] = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(ss, e + 16 * kk, 0, 0));
    }
}

// column m = l % 32 of H_32 at this lane's k positions (the B operands):
// H[k][m] = (-1)^popcount(k & m) with k = 16 kk + 8 (l / 32) + i, whose sign
// is the parity of i & (m % 8) (row m % 8 of H_8 as eight bits), flipped by
// bit 3 of m when l / 32 = 1 and by bit 4 of m when kk = 1
__device__ __forceinline__ void h_operand(int lane, half8v (&hb)[2]) {
    const uint32_t m = uint32_t(lane & 31), g = uint32_t(lane >> 5);
    uint32_t p = ((m & 1u) ? 0xAAu : 0u) ^ ((m & 2u) ? 0xCCu : 0u) ^ ((m & 4u) ? 0xF0u : 0u);
    if (g & (m >> 3) & 1u) p ^= 0xFFu;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const uint32_t q = (kk == 1 && (m & 16u)) ? p ^ 0xFFu : p;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)   // binary16 +-1.0 pairs: 0x3C00 with the sign bit
            w[j] = 0x3C003C00u | (((q >> (2 * j)) & 1u) << 15) | (((q >> (2 * j + 1)) & 1u) << 31);
        hb[kk] = __builtin_bit_cast(half8v, uint4{w[0], w[1], w[2], w[3]});
    }
}

// Rotate one block into out (its 1024 binary16 outputs).
__device__ __forceinline__ void run(const In& in, const half8v (&hb)[2], int lane, uint16_t* out) {
    const int m = lane & 31, g = lane >> 5;
    float16v d = {};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        // a negative sign byte flips the sign bit of its binary16 value: the
        // bytes' top bits moved to bits 15 and 31 of each word
        const uint32_t xw[4] = {in.x[kk].x, in.x[kk].y, in.x[kk].z, in.x[kk].w};
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sm = in.s[kk][j >> 1] & 0x80808080u;
            w[j] = xw[j] ^ __builtin_amdgcn_perm(0u, sm, (j & 1) ? 0x030C020Cu : 0x010C000Cu);
        }
        const half8v a = __builtin_bit_cast(half8v, uint4{w[0], w[1], w[2], w[3]});
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, hb[kk], d, 0, 0, 0);
    }
    // index bits 0, 1, 3, 4 of a: register bits 0, 1, 2, 3
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (!(r & h)) {
                const float u = d[r], v = d[r + h];
                d[r] = u + v;
                d[r + h] = u - v;
            }
    // bit 2 (the lane half): registers r, r + 1 swapped between the halves,
    // after which the lower half holds both values of register r and the
    // upper half both values of register r + 1
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        // (vector elements are copied to scalars before __builtin_bit_cast:
        // applied to a subscripted vector element, it reads element 0)
        const float d0 = d[r], d1 = d[r + 1];
        const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, d0),
                                                         __builtin_bit_cast(uint32_t, d1), false, false);
        const uint32_t s0 = sw[0], s1 = sw[1];
        const float u = __builtin_bit_cast(float, s0), v = __builtin_bit_cast(float, s1);
        const int rr = r + g;
        const int a0 = 8 * (rr >> 2) + (rr & 3);   // a with bit 2 clear
        out[32 * a0 + m] = uint16_t(f2h((u + v) * 0.03125f));
        out[32 * (a0 + 4) + m] = uint16_t(f2h((u - v) * 0.03125f));
    }
}

}  // namespace rot
}  // namespace tl
