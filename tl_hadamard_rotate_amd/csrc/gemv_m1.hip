// Decode GEMV at M = 1 for the 2-bit-slot packing, on the matrix cores:
//
//   y[n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[k]
//
// Ternary multiply-accumulate is additions and subtractions (page "Ternary
// Bonsai 2 27B", section "Что такое тернарная модель"); each 128-group is
// scaled once by its binary16 scale (page "A 27-billion model that fits in
// 8.6 GB", paragraph 2).  At M = 1 a GEMV moves about 0.27 byte per weight, and
// MI355X has only ~5 VALU lane-operations per HBM byte, so the decode may cost
// about one operation per weight.  This kernel spends 10 VALU operations per 16
// weights on it and leaves the multiply-adds to v_mfma_f32_16x16x32_f16.
//
// Decode.  A packed 32-bit word holds 16 digits d = code + 1, digit j at bits
// 2j; its low 16 bits hold digits 0..7, its high 16 bits digits 8..15.  One
// AND of the word (or of the word shifted left by 4 or right by 6) with a
// mask that keeps bits 4-5, 6-7 or 8-9 of both halves leaves a digit pair
// (j, 8 + j) as the binary16 bit patterns d * 2^-20, d * 2^-18 or d * 2^-16
// (subnormal numbers, exact): 10 operations for 16 digits.  The activation
// paired with a digit is stored pre-multiplied by 2^(10 - E), 2^(8 - E) or
// 2^(6 - E) to match (E = exponent of the largest |x| of its column, see
// below), so every product is x * d * 2^(-10 - E).  Bits 0-3 are not used as
// is: products with the two smallest subnormals lose low-order bits in the
// matrix-core sums.  The offset of the digits, sum (d - 1) x = sum d x - sum x,
// is added to each group's sum as -sum_g x * 2^(-10 - E), precomputed with the
// activations.
//
// MFMA use.  Every lane feeds its own activations as A and its own decoded
// digits as B.  Lanes l, l + 16, l + 32, l + 48 form column c = l % 16; the
// diagonal element D[c][c] is the sum of the four lanes' dot products, and the
// rest of D is discarded.  Only 1/16 of each MFMA is useful, which the matrix
// cores afford at M = 1 (one MFMA per 512 weights).
//
// Work split.  One workgroup per CU owns a contiguous slice of the rows.  A
// segment is one row x one 1024-block (256 bytes).  The 16 lanes of a slot
// (four columns) take one segment per step: lane rank u = 4 * (c % 4) + l / 16
// reads bytes [16u, 16u + 16), so a column reads 64 contiguous bytes = two
// groups; lanes l / 16 < 2 hold the first group, the others the second, and
// v_permlane32_swap exchanges words so that each MFMA sees one group only.
// Slots take contiguous runs of segments, block-major, so a slot's
// activations change rarely.  The first two steps' weight loads are in
// flight while the per-lane activation images are built once per workgroup in
// LDS; the rest of a slot's loads follow, all before its first wait on
// weights.  Per-segment sums go to LDS and are added in a fixed order (bitwise
// deterministic).
#include <hip/hip_fp16.h>

#include <type_traits>

#include "rotate_lds.h"
#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
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
    const bool live = t < nb * 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t o = live ? uint32_t((1024 * b + eword_k(u, ep + 2 * h)) * 2) : kOob;
        raw[2 * h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, o, 0, 0));
        raw[2 * h + 1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xs, live ? o + 16 : kOob, 0, 0));
    }
}

__device__ void build_pass(const uint4 (&raw)[4], int nb, int t, uint8_t* img, uint8_t* rec) {
    const bool live = t < nb * 32;
    const int b = live ? t >> 5 : 0;
    const int u = img_u(t);
    const int ep = img_ep(t);
    // largest |x| of the column (bit patterns of non-negative binary16 values
    // order like the values)
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    m = max(m, dpp<kDppHalfMirror>(m));
    int ex = 0;
    if (m >= 0x400u)
        ex = int(m >> 10) - 15;
    else if (m != 0u)
        ex = (31 - __builtin_clz(m)) - 24;
    // pre-scale of in-word position j (its digit decodes to d * 2^(s_j - 24))
    constexpr int kShift[8] = {4, 6, 4, 6, 8, 4, 6, 8};
    float fc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) fc[j] = pow2f(14 - kShift[j] - ex);
    u32x4* dst = reinterpret_cast<u32x4*>(img + b * kImgBlock + u * kImgLane);
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[8] = {raw[2 * h].x, raw[2 * h].y, raw[2 * h].z, raw[2 * h].w,
                               raw[2 * h + 1].x, raw[2 * h + 1].y, raw[2 * h + 1].z,
                               raw[2 * h + 1].w};
        float v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = h2f(w[j] & 0xFFFFu);
            v[2 * j + 1] = h2f(w[j] >> 16);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += v[j];
        // pair j faces digits (j, 8 + j)
        uint32_t out[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = f2h(v[j] * fc[j]) | (f2h(v[8 + j] * fc[j]) << 16);
        const int e = ep + 2 * h;
        if (live) {
            dst[2 * e] = u32x4{out[0], out[1], out[2], out[3]};
            dst[2 * e + 1] = u32x4{out[4], out[5], out[6], out[7]};
        }
    }
    // the column's group sums: over the lane quad, then the other group's
    // from the other quad
    sum += dppf<kDppXor1>(sum);
    sum += dppf<kDppXor2>(sum);
    const float other = dppf<kDppHalfMirror>(sum);
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

__device__ __forceinline__ float pick(const float4v& d, int r) {
    return r == 0 ? d[0] : (r == 1 ? d[1] : (r == 2 ? d[2] : d[3]));
}

// ROT: x is the unrotated activations and signs their signs; the workgroup
// rotates them in LDS first, and workgroup 0 also writes them to x_rot.
template <int FL, bool ROT>
__global__ __launch_bounds__(kThreads) void gemv_m1_slot2_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, const int8_t* signs,
    uint16_t* x_rot, int64_t k, int row_base, int row_rem, int rows_per_chunk,
    void* __restrict__ y, int y_f16) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nb = int(k / kBlock);
    // ROT: [rotated activations nb * 2 KB][transpose scratch, later the images ...]
    uint16_t* xrot = reinterpret_cast<uint16_t*>(smem);
    uint8_t* img = ROT ? smem + nb * 2048 : smem;
    uint8_t* rec = img + nb * kImgBlock;
    float* red = reinterpret_cast<float*>(rec + nb * 4 * kRecBytes);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int slot_in_wave = col >> 2;
    const int ip = lane & 3;                 // column within the slot
    const int u = 4 * ip + q;                // lane rank within the segment
    const int slot = 4 * wave + slot_in_wave;
    const bool diag = q == slot_in_wave;     // this lane holds D[col][col]

    // rows [r0, r0 + rows): row_base rows each, one more for the first row_rem
    const int bid = int(blockIdx.x);
    const int64_t r0 = int64_t(bid) * row_base + min(bid, row_rem);
    const int rows = row_base + (bid < row_rem ? 1 : 0);
    const int64_t row_bytes = k / 4;
    const int64_t groups = k / kGroup;
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + r0 * row_bytes), 0, int(rows * row_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + r0 * groups), 0, int(rows * groups * 2), kRsrcWord3);

    // Per chunk of rows: the slot's segment range [beg, end) (block-major),
    // in flights of FL steps.
    int rc0 = 0, rc = 0, beg = 0, end = 0, flights = 0;
    auto set_chunk = [&](int c0) {
        rc0 = c0;
        rc = min(rows_per_chunk, rows - c0);
        const int segs = rc * nb;
        beg = slot * segs / kSlots;
        end = (slot + 1) * segs / kSlots;
        flights = ((segs + kSlots - 1) / kSlots + FL - 1) / FL;   // workgroup-uniform
    };
    uint4 wv[FL];
    uint32_t sv[FL];
    // every weight and scale load of steps [t_lo, t_hi) of a flight; steps past
    // the slot's end read nothing (out-of-range offsets return zeros)
    auto issue = [&](int f, auto t_lo, auto t_hi) {
        const int f0 = beg + f * FL;
        int b = f0 / rc, r = f0 - (f0 / rc) * rc;
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            const bool ok = f0 + t < end;
            if (t < decltype(t_lo)::value || t >= decltype(t_hi)::value) {
                if (++r == rc) {
                    r = 0;
                    ++b;
                }
                continue;
            }
            const uint32_t wo = ok ? uint32_t((rc0 + r) * row_bytes + 256 * b + 16 * u) : kOob;
            const uint32_t so = ok ? uint32_t(((rc0 + r) * groups + 8 * b + 2 * ip) * 2) : kOob;
            wv[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, wo, 0, 0));
            sv[t] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, so, 0, 0);
            if (++r == rc) {
                r = 0;
                ++b;
            }
        }
    };
    int cur_b = -1;
    half8 a[8];
    float rf = 0.0f, rx = 0.0f, ry = 0.0f;
    auto run = [&](int f) {
        const int f0 = beg + f * FL;
        int b = f0 / rc, r = f0 - (f0 / rc) * rc;
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            const bool ok = f0 + t < end;
            if (ok && b != cur_b) {   // slot-uniform; rare (slots run block-major)
                const uint8_t* src = img + b * kImgBlock + u * kImgLane;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    a[j] = __builtin_bit_cast(
                        half8, *reinterpret_cast<const lds_u32x4*>(lds_addr(src + 16 * j)));
                const float4 rv = *reinterpret_cast<const float4*>(rec + (b * 4 + ip) * kRecBytes);
                rf = rv.x;
                rx = rv.y;
                ry = rv.z;
                cur_b = b;
            }
            const auto p01 = __builtin_amdgcn_permlane32_swap(wv[t].x, wv[t].y, false, false);
            const auto p23 = __builtin_amdgcn_permlane32_swap(wv[t].z, wv[t].w, false, false);
            float4v dx = float4v{0.0f, 0.0f, 0.0f, 0.0f};
            float4v dy = float4v{0.0f, 0.0f, 0.0f, 0.0f};
            dx = mac_eword(p01[0], a[0], a[1], dx);
            dy = mac_eword(p01[1], a[2], a[3], dy);
            dx = mac_eword(p23[0], a[4], a[5], dx);
            dy = mac_eword(p23[1], a[6], a[7], dy);
            const float part = (h2f(sv[t] & 0xFFFFu) * (pick(dx, ip) + rx) +
                                h2f(sv[t] >> 16) * (pick(dy, ip) + ry)) *
                               rf;
            if (diag && ok) red[(r * nb + b) * 4 + ip] = part;
            if (++r == rc) {
                r = 0;
                ++b;
            }
        }
    };
    auto finish_chunk = [&]() {
        lds_barrier();
        for (int r = tid; r < rc; r += kThreads) {
            // fixed order: blocks ascending, the four columns of each block
            const float4* pr = reinterpret_cast<const float4*>(red + r * nb * 4);
            float v = 0.0f;
            int b = 0;
            for (; b + 4 <= nb; b += 4) {
                const float4 p0 = pr[b], p1 = pr[b + 1], p2 = pr[b + 2], p3 = pr[b + 3];
                v = (((v + p0.x) + p0.y) + p0.z) + p0.w;
                v = (((v + p1.x) + p1.y) + p1.z) + p1.w;
                v = (((v + p2.x) + p2.y) + p2.z) + p2.w;
                v = (((v + p3.x) + p3.y) + p3.z) + p3.w;
            }
            for (; b < nb; ++b) {
                const float4 p0 = pr[b];
                v = (((v + p0.x) + p0.y) + p0.z) + p0.w;
            }
            const int64_t o = r0 + rc0 + r;
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
    // Prologue.  The activations are needed first and every workgroup reads
    // them, so they are requested ahead of the weight stream: the loads of the
    // activations, then the first two steps' weights, then the activation images
    // (built by the waves that hold activations), then the rest of the
    // weights.  Requested behind the whole weight stream, the activations
    // would arrive microseconds later (and requesting every step before the
    // images was measured slower).  The activation loads are branch-free
    // buffer loads, so no wave waits for them before its weight loads go out.
    uint4 xraw[4];
    if constexpr (ROT) {
        uint4 sr[2];
        rot::load(x, signs, nb, tid, xraw, sr);
        set_chunk(0);
        issue(0, Zero{}, Head{});
        // the empty asm keeps the rotation below those weight loads
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asm volatile("" : "+v"(xraw[i].x), "+v"(xraw[i].y), "+v"(xraw[i].z), "+v"(xraw[i].w)
                         :
                         : "memory");
        asm volatile("" : "+v"(sr[0].x), "+v"(sr[0].y), "+v"(sr[0].z), "+v"(sr[0].w), "+v"(sr[1].x),
                     "+v"(sr[1].y), "+v"(sr[1].z), "+v"(sr[1].w)
                     :
                     : "memory");
        rot::run(xraw, sr, nb, tid, reinterpret_cast<float*>(img), rot::kScratchFloats, xrot,
                 kBlock);   // nb <= 32 half-waves
        lds_barrier();
        if (blockIdx.x == 0)
            for (int i = tid; i < nb * 128; i += kThreads)
                reinterpret_cast<uint4*>(x_rot)[i] = reinterpret_cast<const uint4*>(xrot)[i];
        load_x_lds(xrot, nb, tid, xraw);
        if (wave * 64 < nb * 32) build_pass(xraw, nb, tid, img, rec);
    } else {
        load_x(x, nb, tid, xraw);
        set_chunk(0);
        issue(0, Zero{}, Head{});
        // the empty asm keeps the image build below those weight loads
#pragma unroll
        for (int i = 0; i < 4; ++i)
            asm volatile("" : "+v"(xraw[i].x), "+v"(xraw[i].y), "+v"(xraw[i].z), "+v"(xraw[i].w)
                         :
                         : "memory");
        if (wave * 64 < nb * 32) build_pass(xraw, nb, tid, img, rec);   // nb * 32 <= kThreads
    }
    lds_barrier();
    issue(0, Head{}, All{});
    run(0);
    for (int f = 1; f < flights; ++f) {
        issue(f, Zero{}, All{});
        run(f);
    }
    finish_chunk();
    for (int c0 = rows_per_chunk; c0 < rows; c0 += rows_per_chunk) {
        set_chunk(c0);
        for (int f = 0; f < flights; ++f) {
            issue(f, Zero{}, All{});
            run(f);
        }
        finish_chunk();
    }
}

int num_cus() {
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    return cus;
}

template <int FL, bool ROT>
hipError_t launch_fl(unsigned grid, size_t lds, const uint8_t* packed, const uint16_t* scales,
                     const uint16_t* x, const int8_t* signs, uint16_t* x_rot, int64_t n,
                     int64_t k, int rpc, void* y, int y_f16, hipStream_t stream) {
    const int base = int(n / grid), rem = int(n % grid);
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemv_m1_slot2_kernel<FL, ROT>),
            hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsLimit));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemv_m1_slot2_kernel<FL, ROT>), dim3(grid), dim3(kThreads), lds, stream,
                       packed, scales, x, signs, x_rot, k, base, rem, rpc, y, y_f16);
    return hipGetLastError();
}

struct M1Plan {
    unsigned grid;
    int rpc;       // rows per chunk
    int steps;     // steps per slot and chunk
    size_t lds;
};

M1Plan m1_plan(int64_t n, int64_t k, bool rot) {
    const int64_t nb = k / kBlock;
    const int64_t grid = n < num_cus() ? n : num_cus();
    const int64_t rows = (n + grid - 1) / grid;                  // largest slice
    int64_t rpc = kMaxSegsPerChunk / nb;
    if (rpc < 1) rpc = 1;
    if (rpc > rows) rpc = rows;
    M1Plan p;
    p.grid = unsigned(grid);
    p.rpc = int(rpc);
    p.steps = int((rpc * nb + kSlots - 1) / kSlots);
    const size_t tail = size_t(nb) * kImgBlock + size_t(nb) * 4 * kRecBytes + size_t(rpc * nb) * 16;
    const size_t scratch = size_t(nb) * rot::kScratchBytes;
    p.lds = rot ? size_t(nb) * 2048 + (tail > scratch ? tail : scratch) : tail;
    return p;
}

template <bool ROT>
hipError_t launch_m1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                     const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k, void* y, int y_f16,
                     hipStream_t stream) {
    const M1Plan p = m1_plan(n, k, ROT);
    switch (p.steps) {
        case 1:
            return launch_fl<1, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 2:
            return launch_fl<2, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 3:
            return launch_fl<3, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 4:
            return launch_fl<4, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 5:
            return launch_fl<5, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 6:
            return launch_fl<6, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 7:
            return launch_fl<7, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        default:
            return launch_fl<8, ROT>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
    }
}

bool m1_fits(int64_t m, int64_t n, int64_t k, bool rot) {
    const int64_t nb = k / kBlock;
    const int64_t grid = n < num_cus() ? n : num_cus();
    const int64_t rows = (n + grid - 1) / grid;
    // one image pass (32 threads per block, one half-wave per rotated block)
    // and 32-bit buffer offsets
    return m == 1 && nb * 32 <= kThreads && m1_plan(n, k, rot).lds <= kLdsLimit &&
           rows * (k / 4) < (int64_t(1) << 31);
}

}  // namespace

bool gemv_m1_slot2_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, false); }

hipError_t launch_gemv_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    return launch_m1<false>(packed, scales, x, nullptr, nullptr, n, k, y, y_f16, stream);
}

bool linear_m1_slot2_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, true); }

hipError_t launch_linear_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                  const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k,
                                  void* y, int y_f16, hipStream_t stream) {
    return launch_m1<true>(packed, scales, x, signs, x_rot, n, k, y, y_f16, stream);
}

}  // namespace tl
