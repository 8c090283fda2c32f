// Decode GEMV for the 1-bit packing (codes -1 and +1, one binary16 scale per
// 128 weights; page "How Prism ML Squeezed a 27B Model Into 3.9 GB", list
// "Two formats ship today"):
//
//   y[m, n] = sum_g S[n, g] * sum_{k in g} (2 b[n, k] - 1) x[m, k]
//           = sum_g S[n, g] * (2 sum_{k in g} b[n, k] x[m, k] - X[m, g])
//
// with b the stored bits and X[m, g] the group sums of the activations.
//
// A workgroup owns 16 weight rows.  A step covers 4 groups: lane 16q + r
// takes row r and group 4s + q of step s, so one 16-byte load per lane reads
// 64 contiguous bytes of each of the 16 rows, and the 16 lanes of a DPP row
// share one group.  The waves of a workgroup split the steps and add their
// partial sums through LDS in a fixed order (bitwise deterministic).
//
// Bits j and j + 16 of a weight dword meet the activation pair
// (x[32d + j], x[32d + j + 16]).  A bit at position 10..14 of a binary16
// (an exponent bit), masked in place, is 0 or one fixed power of two: 2^-14,
// 2^-13, 2^-11, 2^-7 or 2.  Bit pairs 10..14 are masked where they are; pairs
// 5..9 and 0..4 after the dword is shifted up by 5 and 10, pair 15 after it is
// shifted down by 5; each pair then lands on one of the five positions and
// its sum goes to that position's fp32 accumulator, which a group weighs by
// 2 / (its power of two) at the end.  Subnormal masks (bits below 10) are not
// used: v_dot2_f32_f16 adds products with a subnormal operand to the
// accumulator inexactly.
//
// Lane r of a DPP row holds activation pair r of the group's dword d (one
// VGPR per dword, built from two 16-bit loads), and v_dot2c_f32_f16 reads
// pair j for every lane of the row through the DPP row_newbcast:j operand:
// per 2 weights one v_and (shared by all tokens) and one v_dot2c per token.
// X_g is a v_dot2 of the lane's pairs with (1, 1) and a butterfly over the
// row of 16 lanes.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kMaxWaves = 8;
constexpr int kMaxTokens = 16;
constexpr int kRows = 16;   // weight rows per workgroup

// acc_s += the DPP-broadcast pair j of xp times mask m_j, for the 8 bit pairs
// j of one half of a weight dword (pairs 0..7 or 8..15).  Pair j adds to
// accumulator (j mod 5) when j < 15 and to accumulator 0 for j = 15.  The
// leading s_nop covers the DPP read of a VGPR that a VALU wrote just before;
// the trailing one keeps the compiler's next instruction (which may read an
// accumulator the last v_dot2c wrote: measured to read a stale value) out of
// reach.  Inside a block an accumulator is read again 5 instructions after it
// is written at the earliest.
#define TL_DOT(acc, j, m) "v_dot2c_f32_f16_dpp %[" #acc "], %[xp], %[" #m "] row_newbcast:" #j \
                          " row_mask:0xf bank_mask:0xf\n\t"
__device__ __forceinline__ void dot_pairs_lo(float (&a)[5], uint32_t xp, const uint32_t (&m)[16]) {
    asm("s_nop 1\n\t"
        TL_DOT(a0, 0, m0) TL_DOT(a1, 1, m1) TL_DOT(a2, 2, m2) TL_DOT(a3, 3, m3)
        TL_DOT(a4, 4, m4) TL_DOT(a0, 5, m5) TL_DOT(a1, 6, m6) TL_DOT(a2, 7, m7)
        "s_nop 4"
        : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4])
        : [xp] "v"(xp), [m0] "v"(m[0]), [m1] "v"(m[1]), [m2] "v"(m[2]), [m3] "v"(m[3]),
          [m4] "v"(m[4]), [m5] "v"(m[5]), [m6] "v"(m[6]), [m7] "v"(m[7]));
}
__device__ __forceinline__ void dot_pairs_hi(float (&a)[5], uint32_t xp, const uint32_t (&m)[16]) {
    asm("s_nop 1\n\t"
        TL_DOT(a3, 8, m8) TL_DOT(a4, 9, m9) TL_DOT(a0, 10, m10) TL_DOT(a1, 11, m11)
        TL_DOT(a2, 12, m12) TL_DOT(a3, 13, m13) TL_DOT(a4, 14, m14) TL_DOT(a0, 15, m15)
        "s_nop 4"
        : [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4])
        : [xp] "v"(xp), [m8] "v"(m[8]), [m9] "v"(m[9]), [m10] "v"(m[10]), [m11] "v"(m[11]),
          [m12] "v"(m[12]), [m13] "v"(m[13]), [m14] "v"(m[14]), [m15] "v"(m[15]));
}
#undef TL_DOT

// The 16 bit-pair masks of weight dword w: mask j holds bits j and j + 16,
// moved to positions 10 + (j mod 5) (j < 15) or 10 (j = 15) of each half.
__device__ __forceinline__ void pair_masks(uint32_t w, uint32_t (&m)[16]) {
    const uint32_t w10 = w << 10, w5 = w << 5, wr = w >> 5;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        const uint32_t src = j < 5 ? w10 : j < 10 ? w5 : w;
        m[j] = src & (0x00010001u << (10 + j % 5));
    }
    m[15] = wr & 0x04000400u;
}

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }

// 2 / (binary16 value of bit 10 + s alone): 2 / 2^-14, 2 / 2^-13, 2 / 2^-11, 2 / 2^-7, 2 / 2
__device__ constexpr float kSlotWeight[5] = {32768.0f, 16384.0f, 4096.0f, 256.0f, 1.0f};

// MT tokens per pass over the weights (MT = 4: as many passes as needed).
template <int MT>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_bit1_kernel(
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, int m, int64_t n, int64_t k, void* __restrict__ y, int y_f16,
    int waves) {
    __shared__ float part[kMaxWaves * MT * 64];   // partial sums [wave][token][lane]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, q = lane >> 4;   // row in the workgroup, group within a step
    const int groups = int(k / kGroup), steps = groups / 4;
    const int s0 = wave * steps / waves, s1 = (wave + 1) * steps / waves;

    const int64_t n0 = int64_t(blockIdx.x) * kRows;
    const int64_t row = n0 + r < n ? n0 + r : n - 1;   // rows past N redo row N-1
    const uint4* wrow = reinterpret_cast<const uint4*>(packed + row * (k / 8)) + q;
    const uint16_t* srow = scales + row * groups + q;
    const uint16_t* xl = x + 128 * q + r;   // pair r of group 4s + q: x[128 g + 32 d + r], + 16

#pragma unroll 1
    for (int p = 0; p * MT < m; ++p) {
        float acc[MT];
        const uint16_t* xt[MT];   // tokens past m repeat token m - 1 and are never stored
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            acc[t] = 0.0f;
            xt[t] = xl + int64_t(p * MT + t < m ? p * MT + t : m - 1) * k;
        }
        // one step: this lane's bits and scale of group 4s + q, and its
        // activation pairs (d = 0..3) for each token
        struct Step {
            uint4 w;
            uint32_t s;
            uint32_t xp[MT][4];
        };
        auto load_step = [&](int st, Step& b) {
            b.w = wrow[4 * st];
            b.s = srow[4 * st];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint16_t* src = xt[t] + int64_t(st) * 512 + 32 * d;
                    b.xp[t][d] = uint32_t(src[0]) | (uint32_t(src[16]) << 16);
                }
        };
        auto sum_step = [&](const Step& b) {
            const float sc = float(__builtin_bit_cast(_Float16, uint16_t(b.s)));
            const uint32_t wd[4] = {b.w.x, b.w.y, b.w.z, b.w.w};
            float a[MT][5], xs[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                xs[t] = 0.0f;
#pragma unroll
                for (int i = 0; i < 5; ++i) a[t][i] = 0.0f;
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t mk[16];
                pair_masks(wd[d], mk);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    dot_pairs_lo(a[t], b.xp[t][d], mk);
                    dot_pairs_hi(a[t], b.xp[t][d], mk);
                    // the lane's two activations of dword d, added to its share of X
                    xs[t] = __builtin_amdgcn_fdot2(as_h2(b.xp[t][d]), as_h2(0x3C003C00u), xs[t], false);
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                // X of group 4s + q: the 16 lanes of this lane's row of 16
                float xg = xs[t];
                xg += __shfl_xor(xg, 1, 16);
                xg += __shfl_xor(xg, 2, 16);
                xg += __shfl_xor(xg, 4, 16);
                xg += __shfl_xor(xg, 8, 16);
                float ds = a[t][0] * kSlotWeight[0];
#pragma unroll
                for (int i = 1; i < 5; ++i) ds = __builtin_fmaf(a[t][i], kSlotWeight[i], ds);
                acc[t] = __builtin_fmaf(sc, ds - xg, acc[t]);
            }
        };
        // steps in pairs: the next step's loads are in flight while one is summed
        Step bA, bB;
        if (s0 < s1) load_step(s0, bA);
        for (int st = s0; st < s1; st += 2) {
            if (st + 1 < s1) load_step(st + 1, bB);
            sum_step(bA);
            if (st + 1 >= s1) break;
            if (st + 2 < s1) load_step(st + 2, bA);
            sum_step(bB);
        }

        // this pass's tokens: for row r, the 4 groups of a step (lanes r + 16q)
        // and the waves, added in a fixed order
#pragma unroll
        for (int t = 0; t < MT; ++t) part[(wave * MT + t) * 64 + lane] = acc[t];
        __syncthreads();
        for (int t = wave; t < MT && p * MT + t < m; t += waves) {
            if (lane < kRows) {
                float v = 0.0f;
                for (int w = 0; w < waves; ++w)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) v += part[(w * MT + t) * 64 + 16 * qq + lane];
                if (n0 + lane < n) {
                    const int64_t o = int64_t(p * MT + t) * n + n0 + lane;
                    if (y_f16)
                        reinterpret_cast<__half*>(y)[o] = __float2half_rn(v);
                    else
                        reinterpret_cast<float*>(y)[o] = v;
                }
            }
        }
        __syncthreads();
    }
}

// waves per workgroup: the fewest that reach the least number of steps per wave
int waves_for(int64_t k) {
    const int steps = int(k / kGroup) / 4;
    const int most = steps < kMaxWaves ? steps : kMaxWaves;
    const int per = (steps + most - 1) / most;
    int w = most;
    while (w > 1 && (steps + w - 2) / (w - 1) == per) --w;
    return w;
}

template <int MT>
hipError_t launch_mt(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int m,
                     int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    const int waves = waves_for(k);
    hipLaunchKernelGGL(gemv_bit1_kernel<MT>, dim3(unsigned((n + kRows - 1) / kRows)),
                       dim3(64 * waves), 0, stream, packed, scales, x, m, n, k, y, y_f16, waves);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                            int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            hipStream_t stream) {
    const int64_t per = kMaxTokens;   // tokens per launch
    const size_t ysize = y_f16 ? 2 : 4;
    for (int64_t m0 = 0; m0 < m; m0 += per) {
        const int mt = int(m - m0 < per ? m - m0 : per);
        const uint16_t* xc = x + m0 * k;
        void* yc = static_cast<char*>(y) + size_t(m0) * size_t(n) * ysize;
        hipError_t e;
        if (mt == 1)
            e = launch_mt<1>(packed, scales, xc, mt, n, k, yc, y_f16, stream);
        else if (mt == 2)
            e = launch_mt<2>(packed, scales, xc, mt, n, k, yc, y_f16, stream);
        else
            e = launch_mt<4>(packed, scales, xc, mt, n, k, yc, y_f16, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tl
