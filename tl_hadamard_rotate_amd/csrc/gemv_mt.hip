// Decode GEMV for a few tokens (2 <= M <= 16) with the 2-bit-slot packing:
//
//   y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[m, k]
//
// (ternary multiply-accumulate as additions and subtractions: page "Ternary
// Bonsai 2 27B", section "Что такое тернарная модель"; one binary16 scale per
// 128 weights: page "A 27-billion model that fits in 8.6 GB", paragraph 2).
//
// It keeps the M = 1 kernel's digit decode and activation images (m1_decode.h)
// and changes what the matrix-core columns hold, so that the MFMA rows can carry
// tokens.  At M = 1 each of the 16 columns of v_mfma_f32_16x16x32_f16 reads
// different weights of one row and only the diagonal is used.  Here a slot of
// 32 lanes (8 columns x 4 K-quarters) holds a unit of 8 rows x 256 weights: the
// 8 columns are 8 consecutive rows at the SAME 256 positions (one 64-byte
// chunk of each row), and the A row of column i carries token i's activations
// at those positions.  The 8 x 8 diagonal block of D is then [token][row]: one
// MFMA serves 8 tokens for the same decode work and matrix-core instructions as
// one token.  Lane (q, 8s + i) loads row i's bytes [16q, 16q + 16) of the
// chunk, so a column reads 64 contiguous bytes and its lanes q < 2 hold the
// chunk's first group, q >= 2 its second; v_permlane32_swap makes every MFMA
// see one group, exactly as at M = 1.  The byte offset of a lane in the chunk
// (16 * (4 * c' + q), c' = chunk within its 1024-block) is the M = 1 kernel's
// lane rank u = 4 * c' + q, so a token's activation image is the M = 1 image
// and one token's image serves every row of the workgroup.  The two slots of a
// wave take the two chunks of a chunk pair of the same 8 rows, so every load
// instruction reads whole 128-byte lines (64-byte halves read at different
// times were measured 0.2-0.3 us slower per launch).
//
// D rows 8s + 4h .. 8s + 4h + 3 (tokens 4h .. 4h + 3) land in the lanes with
// q = 2s + h.  Those lanes scale the two groups' sums (binary16 scales, the
// digit offset -sum x of the group, the image's power of two) and store the
// four tokens' partial sums of their row and chunk to LDS; the sums are added
// over the chunks in ascending order (bitwise deterministic).
//
// A workgroup holds the images of MT tokens (8, or 4 or 2 when 8 tokens'
// images do not fit in LDS).  With more tokens than that (at most 2 MT), the
// tokens form two groups and both run in one launch: workgroups b and b + 8
// (the same XCD) take the same rows, one group each, so that the second read
// of their weights finds them in that XCD's L2 cache; every workgroup then
// owns twice the rows it would with one group.
//
// The 1-bit packing (codes -1 and +1, bit b = (code + 1) / 2; page "How Prism
// ML Squeezed a 27B Model Into 3.9 GB", list "Two formats ship today") runs
// the same kernel (B1): a lane loads the 8 bytes that hold the same 64
// weights, and each 16 bits of them are spread into the 2-bit-slot word of
// those weights (bit i to bit 2i + 1: digit 2b, which is code + 1 as for
// 2-bit slots); everything after that is shared.
//
// Work split and memory pipeline as at M = 1: one 1024-thread workgroup per CU
// owns a contiguous slice of rows; a wave takes a contiguous run of pair units
// in pair-major order (its activations change only when the chunk pair does);
// the activations are requested first (only by lanes that hold some), then the
// first two steps' weights, then the images are built, then the rest of the
// weights follow, all before the wave's first wait on weights (a ring of
// flights past 7 steps).
#include <hip/hip_fp16.h>

#include <type_traits>

#include "m1_decode.h"
#include "tl_internal.h"

namespace tl {
namespace {

using namespace m1;


constexpr int kUnitRows = 8;                 // rows of a unit (columns of a slot)
constexpr uint32_t kOnes = 0x55555555u;      // 16 digits 1 (codes 0)
constexpr int kTokPad = 16;                  // bytes between token images (LDS bank spread)
constexpr int kRingFlightsMt = 3;            // ring as in the M = 1 kernel: up to 4 flights
constexpr int kRingMaxFLMt = 5;            // 6 does not fit the registers here
// image build rounds of 1024 tasks (32 per token and 1024-block): as many as
// the largest K whose images fit in LDS needs
template <int MT>
constexpr int rounds() { return MT == 2 ? 3 : 2; }

__host__ __device__ constexpr int tok_stride(int nb) { return nb * kImgBlock + kTokPad; }
__host__ __device__ constexpr int rec_tok_bytes(int nb) { return nb * 4 * kRecBytes; }

template <int FL, int MT, bool B1>
__global__ __launch_bounds__(kThreads) void gemv_mt_slot2_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int m, int64_t n,
    int64_t k, int sets, int tgroups, int row_base, int row_rem, int rows_per_chunk,
    void* __restrict__ y, int y_f16) {
    constexpr int V = MT < 4 ? MT : 4;       // tokens per D lane
    // Where the groups' sums of x come from: at 8 tokens from the matrix cores
    // once per chunk (the image build, which runs on every wave, is then the
    // longer part of the prologue); with fewer, from the image build (the
    // extra products slowed the stream more than the sums cost).
    constexpr bool kMfmaOffsets = MT == 8;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nb = int(k / kBlock);
    const int nch = 4 * nb;                  // 256-weight chunks of a row
    const int tstride = tok_stride(nb);
    uint8_t* img = smem;                                    // MT token images
    uint8_t* rec = img + MT * tstride;                      // MT x nb x 4 records
    float* red = reinterpret_cast<float*>(rec + MT * rec_tok_bytes(nb));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int s = col >> 3;                  // slot within the wave: chunk 2p + s of a pair
    const int ip = col & 7;                  // row of the unit; token of the A row
    const int h = q - 2 * s;                 // lanes holding tokens 4h .. 4h + 3 of D
    const bool dlane = (q >> 1) == s && 4 * h < MT;

    // row set and token group of this workgroup: with two groups, workgroups
    // b and b + 8 (b % 16 < 8) take row set (b % 8) + 8 (b / 16), groups 0 and 1
    int bid = int(blockIdx.x), grp = 0;
    if (tgroups == 2) {
        grp = (bid >> 3) & 1;
        bid = (bid & 7) | ((bid >> 4) << 3);
    }
    if (bid >= sets) return;   // padding of the paired grid (whole workgroup)
    const int mt = min(MT, m - grp * MT);
    x += int64_t(grp) * MT * k;
    const int64_t y_tok0 = int64_t(grp) * MT;   // first output row of the group
    const int64_t r0 = int64_t(bid) * row_base + min(bid, row_rem);
    const int rows = row_base + (bid < row_rem ? 1 : 0);
    const int64_t row_bytes = B1 ? k / 8 : k / 4;
    const int64_t groups = k / kGroup;
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + r0 * row_bytes), 0, int(rows * row_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + r0 * groups), 0, int(rows * groups * 2), kRsrcWord3);

    // Per chunk of rows: G groups of 8 rows.  A wave's step is a pair unit:
    // one group of 8 rows at the chunk pair (2p, 2p + 1), slot s taking chunk
    // 2p + s, so the wave reads 128 contiguous bytes (whole cache lines) of
    // each of its 8 rows.  The wave's pair units [beg, end) run pair-major
    // (pair unit = p * G + g), in flights of FL.
    int rc0 = 0, rc = 0, G = 1, beg = 0, end = 0, flights = 0;
    auto set_chunk = [&](int c0) {
        rc0 = c0;
        rc = min(rows_per_chunk, rows - c0);
        G = (rc + kUnitRows - 1) / kUnitRows;
        const int units = (nch / 2) * G;
        beg = wave * units / kWaves;
        end = (wave + 1) * units / kWaves;
        flights = ((units + kWaves - 1) / kWaves + FL - 1) / FL;   // workgroup-uniform
    };
    // a lane's weights of a step: 16 bytes of 2-bit slots or 8 bytes of bits
    using WReg = std::conditional_t<B1, u32x2, uint4>;
    WReg wv[FL];
    uint32_t sv[FL];
    auto load_w = [&](uint32_t wo) -> WReg {
        if constexpr (B1)
            return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wsrc, wo, 0, 0));
        else
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, wo, 0, 0));
    };
    // offsets of step `u` (a unit index) for this lane; out-of-range -> kOob
    auto offsets = [&](int u, int pp, int g, uint32_t& wo, uint32_t& so) {
        const int r = kUnitRows * g + ip;
        const int c = 2 * pp + s;
        const bool ok = u < end && r < rc;
        const int lane_off = B1 ? 32 * c + 8 * q : 64 * c + 16 * q;
        wo = ok ? uint32_t((rc0 + r) * row_bytes + lane_off) : kOob;
        so = ok ? uint32_t(((rc0 + r) * groups + 2 * c) * 2) : kOob;
    };
    auto issue = [&](int f, auto t_lo, auto t_hi) {
        const int f0 = beg + f * FL;
        int c = f0 / G, g = f0 - (f0 / G) * G;
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            if (t >= decltype(t_lo)::value && t < decltype(t_hi)::value) {
                uint32_t wo, so;
                offsets(f0 + t, c, g, wo, so);
                wv[t] = load_w(wo);
                sv[t] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, so, 0, 0);
            }
            if (++g == G) {
                g = 0;
                ++c;
            }
        }
    };

    int cur_c = -1;
    half8 a[8];
    float rf[V], ox[V], oy[V];   // per token: 2^(10+E), digit offsets of the two groups
    // lanes of absent tokens keep zeros (set after the prologue, so that
    // nothing of them is live through it)
    auto clear_a = [&]() {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = half8{};
#pragma unroll
        for (int v = 0; v < V; ++v) rf[v] = ox[v] = oy[v] = 0.0f;
    };

    auto run = [&](int f, auto ring_c) {
        constexpr bool RING = decltype(ring_c)::value;
        const int f0 = beg + f * FL;
        int c = f0 / G, g = f0 - (f0 / G) * G;
        const int g0 = f0 + FL;
        int c2 = g0 / G, gg2 = g0 - (g0 / G) * G;
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            const bool ok = f0 + t < end;
            if (ok && c != cur_c) {   // wave-uniform; once per chunk pair (units run pair-major)
                const int cl = 2 * c + s;   // this slot's chunk
                const int b = cl >> 2, cp = cl & 3;
                if (ip < mt) {
                    const uint8_t* src = img + ip * tstride + b * kImgBlock + (4 * cp + q) * kImgLane;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        a[j] = __builtin_bit_cast(
                            half8, *reinterpret_cast<const lds_u32x4*>(lds_addr(src + 16 * j)));
                }
                if (dlane) {
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const float4 rv = *reinterpret_cast<const float4*>(
                            rec + (4 * h + v) * rec_tok_bytes(nb) + (4 * b + cp) * kRecBytes);
                        rf[v] = rv.x;
                        if constexpr (!kMfmaOffsets) {
                            ox[v] = -rv.y;
                            oy[v] = -rv.z;
                        }
                    }
                }
                if constexpr (kMfmaOffsets) {
                    // the digit offsets (sum of the group's x, image units) from
                    // the matrix cores: the same products as a step whose digits
                    // are all 1 (code 0), so all-zero codes cancel exactly
                    const float4v sx =
                        mac_eword(kOnes, a[4], a[5], mac_eword(kOnes, a[0], a[1], float4v{}));
                    const float4v sy =
                        mac_eword(kOnes, a[6], a[7], mac_eword(kOnes, a[2], a[3], float4v{}));
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        ox[v] = sx[v];
                        oy[v] = sy[v];
                    }
                }
                cur_c = c;
            }
            uint4 w4;
            if constexpr (B1)
                w4 = uint4{spread_bits(wv[t][0], 0), spread_bits(wv[t][0], 1),
                           spread_bits(wv[t][1], 0), spread_bits(wv[t][1], 1)};
            else
                w4 = wv[t];
            const auto p01 = __builtin_amdgcn_permlane32_swap(w4.x, w4.y, false, false);
            const auto p23 = __builtin_amdgcn_permlane32_swap(w4.z, w4.w, false, false);
            float4v dx = float4v{0.0f, 0.0f, 0.0f, 0.0f}, dy = dx;
            dx = mac_eword(p01[0], a[0], a[1], dx);
            dy = mac_eword(p01[1], a[2], a[3], dy);
            dx = mac_eword(p23[0], a[4], a[5], dx);
            dy = mac_eword(p23[1], a[6], a[7], dy);
            const float sa = h2f(sv[t] & 0xFFFFu), sb = h2f(sv[t] >> 16);
            float part[V];
#pragma unroll
            for (int v = 0; v < V; ++v) part[v] = (sa * (dx[v] - ox[v]) + sb * (dy[v] - oy[v])) * rf[v];
            const int r = kUnitRows * g + ip;
            if (dlane && ok && r < rc) {
                float* dst = red + (r * MT + 4 * h) * nch + 2 * c + s;
#pragma unroll
                for (int v = 0; v < V; ++v) dst[v * nch] = part[v];
            }
            if (++g == G) {
                g = 0;
                ++c;
            }
            if constexpr (RING) {
                uint32_t wo, so;
                offsets(g0 + t, c2, gg2, wo, so);
                wv[t] = load_w(wo);
                sv[t] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, so, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (++gg2 == G) {
                    gg2 = 0;
                    ++c2;
                }
            }
        }
    };
    using Plain = std::false_type;
    using Ring = std::true_type;
    auto finish_chunk = [&]() {
        lds_barrier();
        for (int i = tid; i < rc * mt; i += kThreads) {
            const int tk = i / rc, r = i - (i / rc) * rc;
            const float4* pr = reinterpret_cast<const float4*>(red + (r * MT + tk) * nch);
            float v = 0.0f;
            for (int c4 = 0; c4 < nch / 4; ++c4) {   // chunks ascending
                const float4 p = pr[c4];
                v = (((v + p.x) + p.y) + p.z) + p.w;
            }
            const int64_t o = (y_tok0 + tk) * n + r0 + rc0 + r;
            if (y_f16)
                reinterpret_cast<__half*>(y)[o] = __float2half_rn(v);
            else
                reinterpret_cast<float*>(y)[o] = v;
        }
        lds_barrier();
    };

    using Zero = std::integral_constant<int, 0>;
    using Head = std::integral_constant<int, (2 < FL ? 2 : FL)>;
    using All = std::integral_constant<int, FL>;
    const int tasks_per_tok = nb * 32;
    // Prologue: every activation load, then the first two steps' weights,
    // then the images (waves holding activations only).
    uint4 xraw[rounds<MT>()][4];
    const int tasks = mt * tasks_per_tok;
    // one buffer over every token's activations (a per-lane base would make the
    // compiler loop over the distinct descriptors of a wave)
    const __amdgpu_buffer_rsrc_t xsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), 0, mt * nb * 2048, kRsrcWord3);
#pragma unroll
    for (int rd = 0; rd < rounds<MT>(); ++rd) {
        const int tau = rd * kThreads + tid;
        const int tk = tau / tasks_per_tok;
        const int tl = tau - tk * tasks_per_tok;
        const bool live = tau < tasks;
        const int b = tl >> 5, u = img_u(tl), ep = img_ep(tl);
        // lanes without activations issue nothing (even loads that return
        // zeros take the address units' time ahead of the weight loads); their
        // xraw stays unset and unread
        if (live) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const uint32_t o = uint32_t((tk * nb * 1024 + 1024 * b + eword_k(u, ep + 2 * hh)) * 2);
                xraw[rd][2 * hh] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, o, 0, 0));
                xraw[rd][2 * hh + 1] =
                    __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xsrc, o + 16, 0, 0));
            }
        }
    }
    set_chunk(0);
    issue(0, Zero{}, Head{});
    __builtin_amdgcn_sched_barrier(0);   // the image build stays below those weight loads
#pragma unroll
    for (int rd = 0; rd < rounds<MT>(); ++rd) {
        const int tau = rd * kThreads + tid;
        if (rd * kThreads + wave * 64 < tasks) {
            const int tk = tau / tasks_per_tok;
            const bool live = tau < tasks;
            build_pass<!kMfmaOffsets>(xraw[rd], nb, live ? tau - tk * tasks_per_tok : tasks_per_tok,
                       img + (live ? tk : 0) * tstride, rec + (live ? tk : 0) * rec_tok_bytes(nb));
        }
    }
    clear_a();
    lds_barrier();
    if (FL <= kRingMaxFLMt && flights > 1 && flights <= kRingFlightsMt + 1) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vector memory count 0 (see the M = 1 kernel)
        issue(0, Head{}, All{});
#pragma unroll
        for (int f = 0; f < kRingFlightsMt; ++f)
            if (f + 1 < flights) run(f, Ring{});
        run(flights - 1, Plain{});
    } else {
        issue(0, Head{}, All{});
        run(0, Plain{});
        for (int f = 1; f < flights; ++f) {
            issue(f, Zero{}, All{});
            run(f, Plain{});
        }
    }
    finish_chunk();
    for (int c0 = rows_per_chunk; c0 < rows; c0 += rows_per_chunk) {
        set_chunk(c0);
        for (int f = 0; f < flights; ++f) {
            issue(f, Zero{}, All{});
            run(f, Plain{});
        }
        finish_chunk();
    }
}

struct MtPlan {
    unsigned grid;
    int sets;      // row sets (workgroups per token group)
    int groups;    // token groups (1 or 2)
    int mt;        // tokens per group
    int rpc;       // rows per chunk
    int steps;     // steps per wave and row chunk
    size_t lds;
};

size_t fixed_lds(int64_t nb, int mt) {
    return size_t(mt) * size_t(tok_stride(int(nb))) + size_t(mt) * size_t(rec_tok_bytes(int(nb)));
}

// tokens per group: 8, or fewer when 8 images do not fit beside one row of
// partial sums; 0 when not even 2 fit
int pick_mt(int64_t m, int64_t k) {
    const int64_t nb = k / kBlock;
    for (int mt : {8, 4, 2}) {
        if (mt > 2 && mt / 2 >= m) continue;   // the smallest pass that holds m tokens
        const int rd = mt == 2 ? rounds<2>() : (mt == 4 ? rounds<4>() : rounds<8>());
        if (int64_t(mt) * nb * 32 > int64_t(rd) * kThreads) continue;
        if (fixed_lds(nb, mt) + size_t(4 * nb) * mt * 4 <= kLdsLimit) return mt;
    }
    return 0;
}

MtPlan mt_plan(int64_t m, int64_t n, int64_t k) {
    const int64_t nb = k / kBlock;
    MtPlan p{};
    p.mt = pick_mt(m, k);
    if (p.mt == 0) return p;
    // 5..8 tokens in one group of 8, or in two groups of 4 on paired
    // workgroups (each reads the activations of 4 tokens and twice the rows):
    // two groups when a workgroup of one group would read at least three
    // times as many activation bytes (2 m K) as weight bytes (rows K / 4),
    // i.e. rows <= 8 m / 3.  Measured at M = 8: k, v (N = 1024, 8 rows a
    // workgroup) 5.7 -> 5.2 us and o (20 rows) 9.6 -> 8.9 us; q (24 rows)
    // 7.75 -> 8.2 us and q|k|v (32 rows) 8.5 -> 9.1 us, so they keep one group.
    if (p.mt == 8 && m > 4 && m <= 8) {
        const int64_t units1 = (n + kUnitRows - 1) / kUnitRows;
        const int64_t sets1 = units1 < cu_count() ? units1 : cu_count();
        const int64_t rows1 = (n + sets1 - 1) / sets1;
        const bool four_fit = int64_t(4) * nb * 32 <= int64_t(rounds<4>()) * kThreads &&
                              fixed_lds(nb, 4) + size_t(4 * nb) * 4 * 4 <= kLdsLimit;
        if (3 * rows1 <= 8 * m && four_fit) p.mt = 4;
    }
    p.groups = int((m + p.mt - 1) / p.mt);
    // at least a unit of rows per workgroup when there are few rows; with two
    // groups, half the CUs per group and the grid padded to whole 16s (the
    // pairing of workgroups b and b + 8)
    const int64_t units = (n + kUnitRows - 1) / kUnitRows;
    const int64_t cus = p.groups == 2 ? cu_count() / 2 : cu_count();
    const int64_t sets = units < cus ? units : cus;
    const int64_t grid = p.groups == 2 ? 16 * ((sets + 7) / 8) : sets;
    const int64_t rows = (n + sets - 1) / sets;
    const size_t fixed = fixed_lds(nb, p.mt);
    int64_t rpc = int64_t((kLdsLimit - fixed) / (size_t(4 * nb) * p.mt * 4));
    if (rpc > rows) rpc = rows;
    p.grid = unsigned(grid);
    p.sets = int(sets);
    p.rpc = int(rpc);
    const int64_t g = (rpc + kUnitRows - 1) / kUnitRows;
    p.steps = int((2 * nb * g + kWaves - 1) / kWaves);
    p.lds = fixed + size_t(rpc) * size_t(4 * nb) * p.mt * 4;
    return p;
}

template <int FL, int MT, bool B1>
hipError_t launch_fl(const MtPlan& p, const uint8_t* packed, const uint16_t* scales,
                     const uint16_t* x, int m, int64_t n, int64_t k, void* y, int y_f16,
                     hipStream_t stream) {
    const int base = int(n / p.sets), rem = int(n % p.sets);
    const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(gemv_mt_slot2_kernel<FL, MT, B1>), int(kLdsLimit));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_mt_slot2_kernel<FL, MT, B1>), dim3(p.grid), dim3(kThreads), p.lds,
                       stream, packed, scales, x, m, n, k, p.sets, p.groups, base, rem, p.rpc, y,
                       y_f16);
    return hipGetLastError();
}

// every token: one or two groups of at most MT tokens
template <int MT, bool B1>
hipError_t launch_pass(const MtPlan& p, const uint8_t* packed, const uint16_t* scales,
                       const uint16_t* x, int m, int64_t n, int64_t k, void* y, int y_f16,
                       hipStream_t stream) {
    // up to 7 steps a slot: one flight; up to 4 flights of kRingMaxFLMt: a
    // ring; beyond, flights of 7 (8 does not fit the registers)
    if (p.steps > 7 && p.steps <= kRingMaxFLMt * (kRingFlightsMt + 1))
        return launch_fl<kRingMaxFLMt, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
    switch (p.steps) {
        case 1: return launch_fl<1, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        case 2: return launch_fl<2, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        case 3: return launch_fl<3, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        case 4: return launch_fl<4, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        case 5: return launch_fl<5, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        case 6: return launch_fl<6, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
        default: return launch_fl<7, MT, B1>(p, packed, scales, x, m, n, k, y, y_f16, stream);
    }
}

// bytes per weight row: 2-bit slots or 1-bit codes
bool mt_fits(int64_t m, int64_t n, int64_t k, int64_t row_bytes) {
    if (m < 2 || m > 16 || k < kBlock || k % kBlock != 0) return false;
    const MtPlan p = mt_plan(m, n, k);
    if (p.mt == 0 || p.rpc < 1 || p.lds > kLdsLimit) return false;
    // at most two token groups; 32-bit buffer offsets within a workgroup's slice
    const int64_t rows = (n + p.sets - 1) / p.sets;
    return p.groups <= 2 && rows * row_bytes < (int64_t(1) << 31);
}

template <bool B1>
hipError_t launch_mt(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t m,
                     int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    if (!mt_fits(m, n, k, B1 ? k / 8 : k / 4)) return hipErrorInvalidValue;
    const MtPlan p = mt_plan(m, n, k);
    switch (p.mt) {
        case 2: return launch_pass<2, B1>(p, packed, scales, x, int(m), n, k, y, y_f16, stream);
        case 4: return launch_pass<4, B1>(p, packed, scales, x, int(m), n, k, y, y_f16, stream);
        default: return launch_pass<8, B1>(p, packed, scales, x, int(m), n, k, y, y_f16, stream);
    }
}

}  // namespace

bool gemv_mt_slot2_fits(int64_t m, int64_t n, int64_t k) { return mt_fits(m, n, k, k / 4); }

hipError_t launch_gemv_mt_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                                hipStream_t stream) {
    return launch_mt<false>(packed, scales, x, m, n, k, y, y_f16, stream);
}

bool gemv_mt_bit1_fits(int64_t m, int64_t n, int64_t k) { return mt_fits(m, n, k, k / 8); }

hipError_t launch_gemv_mt_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                               int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                               hipStream_t stream) {
    return launch_mt<true>(packed, scales, x, m, n, k, y, y_f16, stream);
}

}  // namespace tl
