// Prefill ternary g128 GEMM on bfloat16 activations (2-bit-slot packing):
//   y[m, n] = sum_g S[n, g] * sum_{k in g} x[m, k] * code[n, k].
// A binary16 scale is not a bfloat16 number, so the scale cannot be folded
// into the weights exactly: the codes enter the bfloat16 matrix cores
// (v_mfma_f32_16x16x32_bf16) as exact -1/0/+1 and each group's fp32 sums are
// multiplied by the group's scale in fp32.  Prompt processing is the
// bottleneck the pages name for slower chips (page "A 27-billion model that
// fits in 8.6 GB", paragraph 4); dense trits and 1-bit codes are rewritten as
// 2-bit slots before this kernel runs.
//
// Tiling: a workgroup of 8 waves computes a 64 x 256 output tile (M x N);
// wave w owns the 32 x 64 sub-tile (w / 4, w % 4), 2 x 4 MFMA tiles, and a
// second set of accumulators for the current group's sums (the reason the
// tile is only 64 rows high: both sets fit in the register file).  K runs in
// steps of BK = 64, half a group, so every MFMA sums within one group,
// through two LDS stages.  Global loads (activations and packed weights) run
// four steps ahead in a ring of registers, so that their latency (an L2 or
// HBM round trip under load) overlaps four steps of MFMAs; during step t the
// MFMAs read stage t % 2 while step t + 1 is written to the other stage
// (activations as loaded, each weight byte expanded to four bfloat16 codes
// through a small LDS table); one barrier per step.
// Both tiles are stored [row][64 values] with the 16-byte chunks of row r
// permuted by c -> c ^ ((r >> 1) & 7), so that the 16 lanes a 128-bit LDS read
// serves per cycle (16 rows, one chunk) hit 16 distinct bank groups.
// Workgroups are mapped so that each XCD (blockIdx % 8) runs a contiguous run
// of tiles, N fastest: concurrent workgroups of an XCD share activation rows
// in that XCD's L2.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "tl_internal.h"

namespace tl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int BM = 64, BN = 256, BK = 64;
constexpr int kMI = BM / 32;                  // 16-row MFMA tiles per wave
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kAStage = BM * BK * 2;          // 8 KB
constexpr int kBStage = BN * BK * 2;          // 32 KB
constexpr int kStage = kAStage + kBStage;
// decode table: entry v = the four bfloat16 codes of byte v (8 bytes); copy c
// of entry v at v * (kCopies * 8) + c * 8.  Lane l reads copy l % kCopies, so
// the 32 lanes one LDS cycle serves never share a bank, whatever bytes they
// look up.
constexpr int kCopies = 32;
constexpr int kLutBytes = 256 * kCopies * 8;  // 64 KB
constexpr int kLds = kLutBytes + 2 * kStage;
static_assert(kLds <= 160 * 1024, "LDS");

// byte offset of 16-byte chunk c of row r in a [rows][64 values] tile
__device__ __forceinline__ uint32_t swz(int r, int c) {
    return uint32_t(r) * 128u + 16u * uint32_t(c ^ ((r >> 1) & 7));
}

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// digit -> bfloat16 bits of d - 1; the invalid digit 3 decodes to 0
__device__ __forceinline__ uint32_t code_bits(uint32_t d) {
    return d == 0u ? 0xBF80u : (d == 2u ? 0x3F80u : 0u);
}

__device__ __forceinline__ void build_lut(uint8_t* lut, int tid) {
    for (int c = tid; c < kLutBytes / 16; c += kThreads) {
        const uint32_t v = uint32_t(c) / (kCopies / 2);   // two 8-byte copies per piece
        const uint32_t lo = code_bits(v & 3u) | (code_bits((v >> 2) & 3u) << 16);
        const uint32_t hi = code_bits((v >> 4) & 3u) | (code_bits((v >> 6) & 3u) << 16);
        reinterpret_cast<uint4*>(lut)[c] = uint4{lo, hi, lo, hi};
    }
}

// Packed bytes of one K step for this thread's weight row and half (32 codes).
struct BRaw {
    uint32_t d[2];
};

__device__ __forceinline__ void load_b(BRaw& r, const uint8_t* prow, int t) {
    const uint2 v = *reinterpret_cast<const uint2*>(prow + 16 * t);
    r.d[0] = v.x;
    r.d[1] = v.y;
}

// LDS address of the table entry for the byte at bit position `shift` of
// word w, in this lane's copy (rep = table base + copy offset)
__device__ __forceinline__ uint32_t lut_off(uint32_t w, int shift, uint32_t rep) {
    return __builtin_amdgcn_ubfe(w, shift, 8) * uint32_t(kCopies * 8) + rep;
}

// the 32 codes of r as 16 bfloat16 pairs
__device__ __forceinline__ void decode_b(const BRaw& r, uint32_t rep, uint32_t (&out)[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint2 e = __builtin_bit_cast(
            uint2, *reinterpret_cast<lds_u32x2*>(lut_off(r.d[i >> 2], 8 * (i & 3), rep)));
        out[2 * i] = e.x;
        out[2 * i + 1] = e.y;
    }
}

__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t m, int64_t n,
    int64_t k, void* __restrict__ y, int y_f16, int tiles_n, int tiles, int chunk) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(smem)));
    const uint32_t st0 = lds0 + kLutBytes;       // stage s at st0 + s * kStage

    // XCD-aware tile order: XCD (blockIdx % 8) takes tiles [xcd * chunk, ...)
    const int tile = int(blockIdx.x & 7) * chunk + int(blockIdx.x >> 3);
    if (tile >= tiles) return;
    const int64_t m0 = int64_t(tile / tiles_n) * BM;
    const int64_t n0 = int64_t(tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ksteps = int(k / BK);
    const int64_t groups = k / kGroup;
    const int64_t row_bytes = k / 4;

    // weight row and half of this thread for the decode: one row per lane,
    // waves 0-3 the first 32 codes of a step, waves 4-7 the last 32
    const int b_row = (wave & 3) * 64 + lane;
    const int hh = wave >> 2;
    const int64_t gn = n0 + b_row < n ? n0 + b_row : n - 1;   // rows past N decode row N-1
    const uint8_t* prow = packed + gn * row_bytes + 8 * hh;
    const uint32_t rep = lds0 + uint32_t(lane & (kCopies - 1)) * 8u;

    // activation row and chunk of this thread (one 16-byte chunk, 64 rows)
    const int ar = tid / 8, ac = tid % 8;
    const int64_t gm = m0 + ar < m ? m0 + ar : m - 1;          // rows past M copy row M-1
    const uint16_t* asrc = x + gm * k + 8 * ac;

    auto load_a = [&](uint4& a, int t) { a = *reinterpret_cast<const uint4*>(asrc + BK * t); };
    auto store_a = [&](const uint4& a, int s) {
        const uint32_t base = st0 + uint32_t(s) * kStage;
        *reinterpret_cast<lds_u32x4*>(base + swz(ar, ac)) = __builtin_bit_cast(u32x4, a);
    };
    auto store_b = [&](const BRaw& r, int s) {
        uint32_t v[16];
        decode_b(r, rep, v);
        const uint32_t base = st0 + uint32_t(s) * kStage + kAStage;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<lds_u32x4*>(base + swz(b_row, 4 * hh + c)) =
                u32x4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
    };

    // Loads run four K steps ahead of their use: step j's raw activations and
    // packed weights sit in ring slot j % 4 until they are written to LDS (the
    // weights decoded) during step j - 1.  K is a multiple of 1024, so the
    // number of steps is a multiple of 16 and the loop below needs no tail;
    // loads past the last step re-read the last step (no branch around any
    // load, so every wait the compiler places is exact).
    uint4 ra[4];
    BRaw rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        load_a(ra[i], i);
        load_b(rb[i], prow, i);
    }
    build_lut(smem, tid);
    lds_barrier();   // the decode table
    store_a(ra[0], 0);
    store_b(rb[0], 0);
    load_a(ra[0], 4);
    load_b(rb[0], prow, 4);
    lds_barrier();

    const int wm = (wave >> 2) * (BM / 2), wn = (wave & 3) * 64;
    float4v acc[kMI][4];
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};
    // this group's sums, and the scales of this lane's four output columns
    // for the current group (loaded at the group's first step)
    float4v grp[kMI][4];
    uint32_t gsc[4] = {0, 0, 0, 0};
    const uint16_t* scol[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t c = n0 + wn + 16 * j + (lane & 15);
        scol[j] = scales + (c < n ? c : n - 1) * groups;   // columns past N read column N-1
    }

    // one K step: MFMAs on stage t & 1, then step t + 1 (ring slot SLOT) to
    // the other stage and step t + 5 loaded into that slot.  t is even for
    // SLOT 1 and 3 (a group's first step) and odd for SLOT 2 and 0.
    auto step = [&](int t, auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr bool kFirst = SLOT == 1 || SLOT == 3;
        const int s = t & 1;
        const uint32_t a_base = st0 + uint32_t(s) * kStage;
        const uint32_t b_base = a_base + kAStage;
        if (kFirst) {
#pragma unroll
            for (int j = 0; j < 4; ++j) gsc[j] = scol[j][t >> 1];
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int c = 4 * ks + (lane >> 4);
            u32x4 af[kMI], bf[4];
#pragma unroll
            for (int i = 0; i < kMI; ++i)
                af[i] = *reinterpret_cast<lds_u32x4*>(a_base + swz(wm + 16 * i + (lane & 15), c));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<lds_u32x4*>(b_base + swz(wn + 16 * j + (lane & 15), c));
#pragma unroll
            for (int i = 0; i < kMI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4v c0 = kFirst && ks == 0 ? float4v{0.f, 0.f, 0.f, 0.f} : grp[i][j];
                    grp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[j]), c0,
                        0, 0, 0);
                }
        }
        if constexpr (!kFirst) {
            // the group is complete: y += S[column, group] * its sums, in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sj = float(__builtin_bit_cast(_Float16, uint16_t(gsc[j])));
#pragma unroll
                for (int i = 0; i < kMI; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(sj, grp[i][j][r], acc[i][j][r]);
            }
        }
        // after the last step this writes a stage nobody reads
        store_a(ra[SLOT], s ^ 1);
        store_b(rb[SLOT], s ^ 1);
        const int t5 = t + 5 < ksteps ? t + 5 : ksteps - 1;
        load_a(ra[SLOT], t5);
        load_b(rb[SLOT], prow, t5);
        lds_barrier();
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    for (int t = 0; t < ksteps; t += 4) {   // step t + 1 is in slot (t + 1) % 4
        step(t, S1{});
        step(t + 1, S2{});
        step(t + 2, S3{});
        step(t + 3, S0{});
    }

    // lane holds D[4 * (lane / 16) + r][lane % 16] of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gm2 = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                const int64_t gcol = n0 + wn + 16 * j + (lane & 15);
                if (gm2 < m && gcol < n) {
                    const float v = acc[i][j][r];
                    if (y_f16)
                        reinterpret_cast<__half*>(y)[gm2 * n + gcol] = __float2half_rn(v);
                    else
                        reinterpret_cast<float*>(y)[gm2 * n + gcol] = v;
                }
            }
}

}  // namespace

hipError_t launch_gemm_bf16_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                  int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                                  hipStream_t stream) {
    if (m < 1 || n < 1 || k < 1024 || k % 1024 != 0) return hipErrorInvalidValue;   // see the loop
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(gemm_bf16_kernel), kLds);
    if (e != hipSuccess) return e;
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t chunk = (tiles + 7) / 8;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3(unsigned(8 * chunk)), dim3(kThreads), size_t(kLds),
                       stream, packed, scales, x, m, n, k, y, y_f16, int(tiles_n), int(tiles),
                       int(chunk));
    return hipGetLastError();
}

}  // namespace tl
