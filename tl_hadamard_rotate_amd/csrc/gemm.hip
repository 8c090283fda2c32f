// Prefill ternary g128 GEMM: y[m, n] = sum_k x[m, k] * code[n, k] * S[n, k/128].
// Weight tiles are dequantised on chip to exact binary16 values code * S (a
// code in {-1, 0, 1} times a binary16 scale is a binary16 number) and the
// contraction runs on the fp16 matrix cores (v_mfma_f32_16x16x32_f16) with
// fp32 accumulation; this is the one dense contraction of the layer.  Prompt
// processing is the bottleneck the pages name for slower chips (page "A
// 27-billion model that fits in 8.6 GB", paragraph 4).
//
// Tiling: a workgroup of 8 waves computes a 128 x 256 output tile (M x N);
// wave w owns the 64 x 64 sub-tile (w / 4, w % 4), 4 x 4 MFMA tiles.  K runs in
// steps of BK = 64 through two LDS stages.  Global loads (activations and
// packed weights) run four steps ahead in a ring of registers, so that their
// latency (an L2 or HBM round trip under load) overlaps four steps of MFMAs;
// during step t the MFMAs read stage t % 2 while step t + 1 is written to the
// other stage (activations as loaded, weights decoded through a small LDS
// table and multiplied by their scale in packed fp16); one barrier per step.
// Both tiles are stored [row][64 halves] with the 16-byte chunks of row r
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

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int BM = 128, BN = 256, BK = 64;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kAStage = BM * BK * 2;          // 16 KB
constexpr int kBStage = BN * BK * 2;          // 32 KB
constexpr int kStage = kAStage + kBStage;
// decode table: TRIT5 entry = five codes in 16 bytes, SLOT2 entry = four codes
// in 8 bytes; copy c of entry v at v * (copies * entry) + c * entry.  Lane l
// reads copy l % copies, so the lanes one LDS cycle serves (256 bytes: 16
// lanes of 16-byte reads, 32 lanes of 8-byte reads) never share a bank,
// whatever bytes they look up.
template <int FMT>
constexpr int entry_bytes() { return FMT == 0 ? 16 : 8; }
template <int FMT>
constexpr int copies() { return FMT == 0 ? 16 : 32; }
template <int FMT>
constexpr int lut_bytes() { return 256 * copies<FMT>() * entry_bytes<FMT>(); }   // 64 KB
template <int FMT>
constexpr int lds_bytes() { return lut_bytes<FMT>() + 2 * kStage; }
static_assert(lds_bytes<0>() <= 160 * 1024 && lds_bytes<1>() <= 160 * 1024, "LDS");

// byte offset of 16-byte chunk c of row r in a [rows][64 halves] tile
__device__ __forceinline__ uint32_t swz(int r, int c) {
    return uint32_t(r) * 128u + 16u * uint32_t(c ^ ((r >> 1) & 7));
}

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// digit -> bits of (d - 1) as binary16 (or bfloat16); an invalid digit decodes to 0
template <bool BF16>
__device__ __forceinline__ uint32_t code_bits(uint32_t d) {
    if (BF16) return d == 0u ? 0xBF80u : (d == 2u ? 0x3F80u : 0u);
    return d == 0u ? 0xBC00u : (d == 2u ? 0x3C00u : 0u);
}

template <int FMT, bool BF16>
__device__ __forceinline__ void build_lut(uint8_t* lut, int tid) {
    for (int c = tid; c < lut_bytes<FMT>() / 16; c += kThreads) {
        if (FMT == 0) {
            const uint32_t v = uint32_t(c) / copies<FMT>();   // one 16-byte entry per piece
            uint32_t h[5] = {0, 0, 0, 0, 0};
            if (v < 243) {
                uint32_t r = v;
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    h[i] = code_bits<BF16>(r % 3u);
                    r /= 3u;
                }
            }
            reinterpret_cast<uint4*>(lut)[c] =
                uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u};
        } else {
            const uint32_t v = uint32_t(c) / (copies<FMT>() / 2);   // two 8-byte copies per piece
            const uint32_t lo = code_bits<BF16>(v & 3u) | (code_bits<BF16>((v >> 2) & 3u) << 16);
            const uint32_t hi =
                code_bits<BF16>((v >> 4) & 3u) | (code_bits<BF16>((v >> 6) & 3u) << 16);
            reinterpret_cast<uint4*>(lut)[c] = uint4{lo, hi, lo, hi};
        }
    }
}

// binary16 pair times the scale pair (exact: codes are -1, 0, 1)
__device__ __forceinline__ uint32_t scale_pair(uint32_t codes, half2v s2) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, codes) * s2);
}

// Packed bytes of one K step for this thread's weight row and half (32 codes).
struct BRaw {
    uint32_t d[7];    // TRIT5: the group's 26 bytes from byte (26g & 3); SLOT2: d[0..1]
    uint32_t s;       // the row's scales of groups (g & ~1, g | 1): a whole
                      // register, so a load into one ring slot never waits on
                      // a register shared with another
};

template <int FMT>
__device__ __forceinline__ void load_b(BRaw& r, const uint8_t* prow, const uint16_t* srow, int t) {
    const int g = t >> 1;
    if (FMT == 0) {
        // 28 bytes from the dword holding the group's first byte: in bounds
        // for every group (the last group of a row starts at 2 mod 4)
        const uint8_t* a = prow + 26 * g - ((26 * g) & 3);
        const uint4 lo = *reinterpret_cast<const uint4*>(a);
        const uint4 hi = *reinterpret_cast<const uint4*>(a + 12);
        r.d[0] = lo.x; r.d[1] = lo.y; r.d[2] = lo.z; r.d[3] = lo.w;
        r.d[4] = hi.y; r.d[5] = hi.z; r.d[6] = hi.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(prow + 16 * t);
        r.d[0] = v.x;
        r.d[1] = v.y;
    }
    r.s = *reinterpret_cast<const uint32_t*>(srow + (g & ~1));   // rows hold 8k groups
}

// LDS address of the table entry for the byte at bit position `shift` of
// word w, in this lane's copy (rep = table base + copy offset)
template <int FMT>
__device__ __forceinline__ uint32_t lut_off(uint32_t w, int shift, uint32_t rep) {
    return __builtin_amdgcn_ubfe(w, shift, 8) * uint32_t(copies<FMT>() * entry_bytes<FMT>()) + rep;
}

// TRIT5: codes (c, c + 1) of a group from the entries of the byte holding c
// and of the next byte
__device__ __forceinline__ uint32_t code_pair(int digit, const uint4& e, const uint4& en) {
    switch (digit) {
        case 0: return e.x;
        case 1: return __builtin_amdgcn_perm(e.y, e.x, 0x05040302u);   // e.x hi, e.y lo
        case 2: return e.y;
        case 3: return __builtin_amdgcn_perm(e.z, e.y, 0x05040302u);   // e.y hi, e.z lo
        default: return __builtin_amdgcn_perm(en.x, e.z, 0x05040100u); // e.z lo, en.x lo
    }
}

// Decode 32 codes (TRIT5 codes [cs, cs + 32) of the group; the group's byte i
// sits at byte i + o of r.d) into 16 scaled binary16 pairs.
template <int CS, int O>
__device__ __forceinline__ void decode_t5(const BRaw& r, uint32_t rep, half2v s2, uint32_t (&out)[16]) {
    constexpr int b_lo = CS / 5, b_hi = (CS + 31) / 5;
    uint4 e[b_hi - b_lo + 1];
#pragma unroll
    for (int b = b_lo; b <= b_hi; ++b) {
        const int p = b + O;
        e[b - b_lo] = __builtin_bit_cast(
            uint4, *reinterpret_cast<lds_u32x4*>(lut_off<0>(r.d[p >> 2], 8 * (p & 3), rep)));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = CS + 2 * i;
        const int b = c / 5 - b_lo;
        out[i] = scale_pair(code_pair(c % 5, e[b], e[b + (c % 5 == 4 ? 1 : 0)]), s2);
    }
}

// BF16: the codes as bfloat16 -1/0/+1, unscaled (the scale is applied to the
// fp32 sums of each group); otherwise code * S in binary16
template <int FMT, bool BF16>
__device__ __forceinline__ void decode_b(const BRaw& r, int t, int hh, uint32_t rep,
                                         uint32_t (&out)[16]) {
    const uint16_t sh = uint16_t(r.s >> (16 * ((t >> 1) & 1)));   // wave-uniform select
    const half2v s2 = half2v{__builtin_bit_cast(_Float16, sh), __builtin_bit_cast(_Float16, sh)};
    if (FMT == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint2 e = __builtin_bit_cast(
                uint2, *reinterpret_cast<lds_u32x2*>(lut_off<1>(r.d[i >> 2], 8 * (i & 3), rep)));
            out[2 * i] = BF16 ? e.x : scale_pair(e.x, s2);
            out[2 * i + 1] = BF16 ? e.y : scale_pair(e.y, s2);
        }
    } else {
        // wave-uniform: which 32 codes of the group, and the group's byte offset
        const int cs = 64 * (t & 1) + 32 * hh;
        const int o = (26 * (t >> 1)) & 3;
        switch (cs + o) {
            case 0: decode_t5<0, 0>(r, rep, s2, out); break;
            case 2: decode_t5<0, 2>(r, rep, s2, out); break;
            case 32: decode_t5<32, 0>(r, rep, s2, out); break;
            case 34: decode_t5<32, 2>(r, rep, s2, out); break;
            case 64: decode_t5<64, 0>(r, rep, s2, out); break;
            case 66: decode_t5<64, 2>(r, rep, s2, out); break;
            case 96: decode_t5<96, 0>(r, rep, s2, out); break;
            default: decode_t5<96, 2>(r, rep, s2, out); break;
        }
    }
}

// Activations of one K step for this thread: row ar of the tile, 16-byte
// chunks ac and ac + 1 (32 contiguous bytes; four threads per 128-byte row).
struct ARaw {
    uint4 v[2];
};

// BF16: x is bfloat16, the codes enter the matrix cores as bfloat16 -1/0/+1
// and each group's fp32 sums are multiplied by their column's scale (the
// K step of 64 is half a group, so every MFMA sums within one group).  The
// group's sums need a second set of accumulators, so the tile is 64 x 256
// (a wave owns 32 x 64) to stay within 256 registers.
template <bool BF16>
constexpr int tile_m() { return BF16 ? 64 : BM; }

template <int FMT, bool BF16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t m, int64_t n,
    int64_t k, void* __restrict__ y, int y_f16, int tiles_n, int tiles, int chunk) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(smem)));
    const uint32_t st0 = lds0 + lut_bytes<FMT>();       // stage s at st0 + s * kStage

    // XCD-aware tile order: XCD (blockIdx % 8) takes tiles [xcd * chunk, ...)
    const int tile = int(blockIdx.x & 7) * chunk + int(blockIdx.x >> 3);
    if (tile >= tiles) return;
    constexpr int kBM = tile_m<BF16>(), kMI = kBM / 32;   // kMI: 16-row MFMA tiles per wave
    const int64_t m0 = int64_t(tile / tiles_n) * kBM;
    const int64_t n0 = int64_t(tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ksteps = int(k / BK);
    const int64_t groups = k / kGroup;
    const int64_t row_bytes = FMT == 0 ? groups * kTrit5GroupBytes : k / 4;

    // weight row and half of this thread for the decode: one row per lane,
    // waves 0-3 the first 32 codes of a step, waves 4-7 the last 32
    const int b_row = (wave & 3) * 64 + lane;
    const int hh = wave >> 2;
    const int64_t gn = n0 + b_row < n ? n0 + b_row : n - 1;   // rows past N decode row N-1
    const uint8_t* prow = packed + gn * row_bytes + (FMT == 1 ? 8 * hh : 0);
    const uint16_t* srow = scales + gn * groups;
    const uint32_t rep = lds0 + uint32_t(lane & (copies<FMT>() - 1)) * uint32_t(entry_bytes<FMT>());

    // activation row and chunks of this thread
    // (BF16: one chunk per thread over 64 rows, else two over 128 rows)
    constexpr int kAChunks = kBM / 64;
    const int ar = tid / (8 / kAChunks), ac = kAChunks * (tid % (8 / kAChunks));
    const int64_t gm = m0 + ar < m ? m0 + ar : m - 1;          // rows past M copy row M-1
    const uint16_t* asrc = x + gm * k + 8 * ac;

    auto load_a = [&](ARaw& a, int t) {
        const uint4* p = reinterpret_cast<const uint4*>(asrc + BK * t);
#pragma unroll
        for (int c = 0; c < kAChunks; ++c) a.v[c] = p[c];
    };
    auto store_a = [&](const ARaw& a, int s) {
        const uint32_t base = st0 + uint32_t(s) * kStage;
#pragma unroll
        for (int c = 0; c < kAChunks; ++c)
            *reinterpret_cast<lds_u32x4*>(base + swz(ar, ac + c)) = __builtin_bit_cast(u32x4, a.v[c]);
    };
    auto store_b = [&](const BRaw& r, int t, int s) {
        uint32_t v[16];
        decode_b<FMT, BF16>(r, t, hh, rep, v);
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
    ARaw ra[4];
    BRaw rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        load_a(ra[i], i);
        load_b<FMT>(rb[i], prow, srow, i);
    }
    build_lut<FMT, BF16>(smem, tid);
    lds_barrier();   // the decode table
    store_a(ra[0], 0);
    store_b(rb[0], 0, 0);
    load_a(ra[0], 4);
    load_b<FMT>(rb[0], prow, srow, 4);
    lds_barrier();

    const int wm = (wave >> 2) * (kBM / 2), wn = (wave & 3) * 64;
    float4v acc[kMI][4];
#pragma unroll
    for (int i = 0; i < kMI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};
    // BF16: this group's sums, and the scales of this lane's four output
    // columns for the current group (loaded at the group's first step)
    float4v grp[BF16 ? kMI : 1][BF16 ? 4 : 1];
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
        if (BF16 && kFirst) {
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
                    if constexpr (BF16) {
                        const float4v c0 = kFirst && ks == 0 ? float4v{0.f, 0.f, 0.f, 0.f}
                                                             : grp[i][j];
                        grp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[j]),
                            c0, 0, 0, 0);
                    } else {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(half8, af[i]), __builtin_bit_cast(half8, bf[j]),
                            acc[i][j], 0, 0, 0);
                    }
                }
        }
        if constexpr (BF16 && !kFirst) {
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
        const int t1 = t + 1 < ksteps ? t + 1 : ksteps - 1;
        store_a(ra[SLOT], s ^ 1);
        store_b(rb[SLOT], t1, s ^ 1);
        const int t5 = t + 5 < ksteps ? t + 5 : ksteps - 1;
        load_a(ra[SLOT], t5);
        load_b<FMT>(rb[SLOT], prow, srow, t5);
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

template <int FMT, bool BF16 = false>
hipError_t launch(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t m,
                  int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel<FMT, BF16>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 lds_bytes<FMT>());
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t tiles_m = (m + tile_m<BF16>() - 1) / tile_m<BF16>(), tiles_n = (n + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t chunk = (tiles + 7) / 8;
    hipLaunchKernelGGL((gemm_kernel<FMT, BF16>), dim3(unsigned(8 * chunk)), dim3(kThreads),
                       size_t(lds_bytes<FMT>()), stream, packed, scales, x, m, n, k, y, y_f16,
                       int(tiles_n), int(tiles), int(chunk));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    if (m < 1 || n < 1 || k < 1024 || k % 1024 != 0) return hipErrorInvalidValue;   // see the loop
    if (fmt == 1 && gemm_slot2_fits(m, n, k))
        return launch_gemm_slot2(packed, scales, x, m, n, k, y, y_f16, stream);
    if (fmt == 0 && gemm_slot2_fits(m, n, k)) {
        // dense trits: rewritten as 2-bit slots once per call (one pass over
        // the weights, small next to the product) for the same GEMM
        void* slot2 = nullptr;
        hipError_t e = workspace(kWorkspaceSlot2, stream, size_t(n) * size_t(k / 4), &slot2);
        if (e != hipSuccess) return e;
        if ((e = launch_trit5_to_slot2(packed, n, k, static_cast<uint8_t*>(slot2), stream)) != hipSuccess)
            return e;
        return launch_gemm_slot2(static_cast<const uint8_t*>(slot2), scales, x, m, n, k, y, y_f16, stream);
    }
    if (fmt == 2) {
        // 1-bit codes: rewritten as 2-bit slots (digits 0 and 2) once per call
        void* slot2 = nullptr;
        hipError_t e = workspace(kWorkspaceSlot2, stream, size_t(n) * size_t(k / 4), &slot2);
        if (e != hipSuccess) return e;
        if ((e = launch_bit1_to_slot2(packed, n, k, static_cast<uint8_t*>(slot2), stream)) != hipSuccess)
            return e;
        const uint8_t* s2 = static_cast<const uint8_t*>(slot2);
        return gemm_slot2_fits(m, n, k) ? launch_gemm_slot2(s2, scales, x, m, n, k, y, y_f16, stream)
                                        : launch<1>(s2, scales, x, m, n, k, y, y_f16, stream);
    }
    return fmt == 0 ? launch<0>(packed, scales, x, m, n, k, y, y_f16, stream)
                    : launch<1>(packed, scales, x, m, n, k, y, y_f16, stream);
}

hipError_t launch_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int fmt,
                            const uint16_t* x, int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            hipStream_t stream) {
    if (m < 1 || n < 1 || k < 1024 || k % 1024 != 0) return hipErrorInvalidValue;
    const uint8_t* s2 = packed;
    if (fmt != 1) {
        // dense trits and 1-bit codes: rewritten as 2-bit slots once per call
        void* ws = nullptr;
        hipError_t e = workspace(kWorkspaceSlot2, stream, size_t(n) * size_t(k / 4), &ws);
        if (e != hipSuccess) return e;
        e = fmt == 0 ? launch_trit5_to_slot2(packed, n, k, static_cast<uint8_t*>(ws), stream)
                     : launch_bit1_to_slot2(packed, n, k, static_cast<uint8_t*>(ws), stream);
        if (e != hipSuccess) return e;
        s2 = static_cast<const uint8_t*>(ws);
    }
    return launch<1, true>(s2, scales, x, m, n, k, y, y_f16, stream);
}

}  // namespace tl
