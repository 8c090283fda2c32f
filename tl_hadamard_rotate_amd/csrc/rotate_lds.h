// Signed 1024-block Hadamard rotation of one activation row into LDS, for
// the GEMV kernels that rotate in their prologue (tl_linear at M = 1):
//
//   x'[1024 b + i] = (1/32) sum_j H[i, j] s[1024 b + j] x[1024 b + j]
//
// (page "OpenBonsai", section "How it works", step 1; page "A 27-billion
// model that fits in 8.6 GB", paragraphs 2 and 3: the rotation folded into
// the weights has to be applied to the activations at run time.)
//
// Half-wave hw (32 lanes) rotates block hw: lane j loads elements
// [32j, 32j + 32) and their signs, does the butterflies of index bits 0-4 in
// registers, transposes through LDS (row stride 33 floats: conflict-free both
// ways), does bits 5-9 in registers, and writes (1/32) * result, rounded once
// to binary16, to the block's output.  fp32 throughout, 10 butterfly levels per
// output, like tl_hadamard_rotate (the summation order differs, so the two
// agree to within that bound rather than bit for bit).
#pragma once

#include "tl_internal.h"

namespace tl {
namespace rot {

constexpr int kScratchFloats = 32 * 33;          // transpose scratch per block
constexpr int kScratchBytes = kScratchFloats * 4;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOob = 0x80000000u;           // offset past every range: loads return 0

__device__ __forceinline__ float h2f(uint32_t h) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h)));
}
__device__ __forceinline__ uint32_t f2h(float f) {
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(f)));
}

// The loads of thread t: x[1024 hw + 32 j ...] (64 bytes) and its signs (32
// bytes).  Lanes past the last block issue nothing (loads that return zeros
// still take the address units' time ahead of what follows) and leave xr and
// sr unset; run() does nothing for them.
__device__ __forceinline__ void load(const uint16_t* x, const int8_t* signs, int nb, int t,
                                     uint4 (&xr)[4], uint4 (&sr)[2]) {
    const int hw = t >> 5, j = t & 31;
    const __amdgpu_buffer_rsrc_t xs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, nb * 2048, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ss =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, nb * 1024, kRsrcWord3);
    if (hw >= nb) return;
    const uint32_t xo = uint32_t((1024 * hw + 32 * j) * 2);
    const uint32_t so = uint32_t(1024 * hw + 32 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, xo + 16 * i, 0, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ss, so + 16 * i, 0, 0));
}

template <int H>
__device__ __forceinline__ void butterfly(float (&v)[32]) {
#pragma unroll
    for (int i = 0; i < 32; ++i)
        if (!(i & H)) {
            const float a = v[i], b = v[i + H];
            v[i] = a + b;
            v[i + H] = a - b;
        }
}

__device__ __forceinline__ void butterflies(float (&v)[32]) {
    butterfly<1>(v);
    butterfly<2>(v);
    butterfly<4>(v);
    butterfly<8>(v);
    butterfly<16>(v);
}

// Rotate block hw = t / 32 (whole half-waves; hw >= nb do nothing).  Its
// transpose scratch is kScratchFloats floats at scratch + hw * scratch_stride
// (floats), its 1024 binary16 outputs go to out + hw * out_stride (halves).
// The output of a block may overlap its own scratch (each half-wave reads its
// scratch back before it writes its output), not another block's.
__device__ __forceinline__ void run(const uint4 (&xr)[4], const uint4 (&sr)[2], int nb, int t,
                                    float* scratch, int scratch_stride, uint16_t* out,
                                    int out_stride) {
    const int hw = t >> 5, j = t & 31;
    if (hw >= nb) return;
    const uint32_t xw[16] = {xr[0].x, xr[0].y, xr[0].z, xr[0].w, xr[1].x, xr[1].y, xr[1].z, xr[1].w,
                             xr[2].x, xr[2].y, xr[2].z, xr[2].w, xr[3].x, xr[3].y, xr[3].z, xr[3].w};
    const uint32_t sw[8] = {sr[0].x, sr[0].y, sr[0].z, sr[0].w, sr[1].x, sr[1].y, sr[1].z, sr[1].w};
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        // a negative sign byte flips the sign bit of the fp32 value
        const uint32_t neg = ((sw[i >> 2] >> (8 * (i & 3) + 7)) & 1u) << 31;
        v[i] = __builtin_bit_cast(
            float, __builtin_bit_cast(uint32_t, h2f((xw[i >> 1] >> (16 * (i & 1))) & 0xFFFFu)) ^ neg);
    }
    butterflies(v);
    float* row = scratch + hw * scratch_stride;
#pragma unroll
    for (int i = 0; i < 32; ++i) row[j * 33 + i] = v[i];
    // the same wave wrote the rows: its LDS operations complete in order
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = row[i * 33 + j];   // element 32 i + j
    butterflies(v);
    uint16_t* o = out + hw * out_stride + j;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[32 * i] = uint16_t(f2h(v[i] * 0.03125f));
}

}  // namespace rot
}  // namespace tl
