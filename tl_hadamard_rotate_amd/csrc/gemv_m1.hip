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
// The four slots of a wave take four consecutive rows of the same block per
// step (a unit); a wave takes a contiguous run of units, block-major, so its
// activations change rarely, and every address of a step is a wave-uniform
// offset plus a per-lane constant.  The first two steps' weight loads are in
// flight while the per-lane activation images are built once per workgroup in
// LDS; the rest of a slot's loads follow, all before its first wait on
// weights.  Per-segment sums go to LDS and are added in a fixed order (bitwise
// deterministic).
#include <hip/hip_fp16.h>

#include <type_traits>

#include "m1_decode.h"
#include "rotate_lds.h"
#include "tl_internal.h"

namespace tl {
namespace {

using namespace m1;

constexpr int kRingFlights = 3;   // flights of a chunk streamed as a ring: up to 4 in all
constexpr int kRingMaxFL = 6;     // flight length of the ring (8 does not fit the registers)
// cache policy of the weight and scale loads: read once per call, streamed
// (nontemporal) so that they do not push the activations out of the caches
constexpr int kNonTemporal = 2;

// ROT: x is the unrotated activations and signs their signs; the workgroup
// rotates them in LDS first, and workgroup 0 also writes them to x_rot.
// B1: the 1-bit packing (codes -1 and +1, bit b = (code + 1) / 2, 16 bytes
// per 128 weights): a lane loads the 8 bytes that hold the 64 weights it
// would read as 16 bytes of 2-bit slots, and each 16 bits of them are
// spread into the 2-bit-slot word of the same weights (digit 2b = code + 1);
// everything after that is the 2-bit-slot kernel.
template <int FL, bool ROT, bool B1>
__global__ __launch_bounds__(kThreads) void gemv_m1_slot2_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, const int8_t* signs,
    uint16_t* x_rot, int64_t k, int row_base, int row_rem, int rows_per_chunk,
    void* __restrict__ y, int y_f16) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nb = int(k / kBlock);
    // ROT: [rotated activations nb * 2 KB][images ...]
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
    const bool diag = q == slot_in_wave;     // this lane holds D[col][col]

    // rows [r0, r0 + rows): row_base rows each, one more for the first row_rem
    const int bid = int(blockIdx.x);
    const int64_t r0 = int64_t(bid) * row_base + min(bid, row_rem);
    const int rows = row_base + (bid < row_rem ? 1 : 0);
    const int64_t row_bytes = B1 ? k / 8 : k / 4;
    constexpr int kLaneBytes = B1 ? 8 : 16;          // a lane's bytes of a step
    constexpr int kSegBytes = 16 * kLaneBytes;       // a row's bytes of a 1024-block
    const int64_t groups = k / kGroup;
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + r0 * row_bytes), 0, int(rows * row_bytes), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ssrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales + r0 * groups), 0, int(rows * groups * 2), kRsrcWord3);

    // Per chunk of rows, work in units of four rows x one 1024-block (one row
    // per slot of a wave, the same block for the wave's four slots),
    // block-major; wave w takes units [vb, ve) in flights of FL steps.  The
    // unit, its block and its first row are wave-uniform, so every address
    // of a step is a scalar offset plus a per-lane constant (no per-step
    // vector arithmetic).  A block's last unit starts at row rc - 4 (its rows
    // overlap the unit before: those partial sums are computed twice and
    // written twice with the same bits); with fewer than four rows the slots
    // past the last row repeat it.  Steps past a wave's last unit repeat that
    // unit the same way.
    int rc0 = 0, rc = 0, U = 1, vb = 0, ve = 0, flights = 0;
    uint32_t w_lane = 0, s_lane = 0;
    int red_lane = 0;
    // a step's unit: index v, block b, unit j of the block (all wave-uniform)
    struct Cur {
        int v, b, j;
    };
    Cur first{0, 0, 0};  // the wave's first unit of the chunk
    Cur last{0, 0, 0};   // the unit that steps past the wave's last one repeat
    // v / U by a float reciprocal and one correction (v < 2^20): a scalar
    // integer division is a long sequence of scalar instructions, which the
    // four SIMDs of a CU share
    auto cur_at = [&](int v) {
        int b = int(float(v) * __builtin_amdgcn_rcpf(float(U)));
        if ((b + 1) * U <= v)
            ++b;
        else if (b * U > v)
            --b;
        return Cur{v, b, v - b * U};
    };
    // (the block passes through readfirstlane: else the compiler may form its
    // increment as a vector add with carry, and each load offset made from
    // it becomes a loop over the lanes' distinct values)
    auto cur_next = [&](Cur c) {
        ++c.v;
        if (++c.j == U) {
            c.j = 0;
            ++c.b;
        }
        c.b = __builtin_amdgcn_readfirstlane(c.b);
        return c;
    };
    auto advance = [&](Cur c) {
#pragma unroll
        for (int t = 0; t < FL; ++t) c = cur_next(c);
        return c;
    };
    auto eff = [&](const Cur& c) { return c.v < ve ? c : last; };
    auto set_chunk = [&](int c0) {
        rc0 = c0;
        rc = min(rows_per_chunk, rows - c0);
        U = (rc + 3) / 4;
        const int units = U * nb;
        vb = wave * units / kWaves;
        ve = (wave + 1) * units / kWaves;
        last = cur_at(ve > vb ? ve - 1 : units - 1);
        first = cur_at(vb);
        flights = ((units + kWaves - 1) / kWaves + FL - 1) / FL;   // workgroup-uniform
        const int s_eff = min(slot_in_wave, rc - 1);
        w_lane = uint32_t(s_eff * int(row_bytes) + kLaneBytes * u);
        s_lane = uint32_t((s_eff * int(groups) + 2 * ip) * 2);
        red_lane = s_eff * nb * 4 + ip;
    };
    auto row0 = [&](const Cur& c) { return rc < 4 ? 0 : min(4 * c.j, rc - 4); };
    // Step t of a flight: its weights and scales in registers, and (scalar)
    // its block and the offset of its partial sums in red, set when its loads
    // are issued so that consuming it takes no unit arithmetic.
    using WReg = std::conditional_t<B1, u32x2, uint4>;
    WReg wv[FL];
    uint32_t sv[FL];
    int sb[FL], sro[FL];
    auto load_step = [&](int t, const Cur& c) {
        const Cur e = eff(c);
        const int r0e = row0(e);
        const int r = rc0 + r0e;
        const uint32_t wo = uint32_t(r * int(row_bytes) + kSegBytes * e.b);
        if constexpr (B1)
            wv[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wsrc, w_lane, wo, kNonTemporal));
        else
            wv[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, w_lane, wo, kNonTemporal));
        sv[t] = __builtin_amdgcn_raw_buffer_load_b32(ssrc, s_lane,
                                                     uint32_t((r * int(groups) + 8 * e.b) * 2), kNonTemporal);
        sb[t] = e.b;
        sro[t] = (r0e * nb + e.b) * 4;
    };
    // every weight and scale load of steps [t_lo, t_hi) of the flight starting at c
    auto issue = [&](Cur c, auto t_lo, auto t_hi) {
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            if (t >= decltype(t_lo)::value && t < decltype(t_hi)::value) load_step(t, c);
            c = cur_next(c);
        }
    };
    int cur_b = -1;
    half8 a[8];
    float rf = 0.0f, rx = 0.0f, ry = 0.0f;
    // The flight whose loads were issued last.  With RING, as soon as step t
    // is consumed its registers receive step t of the next flight (starting
    // at c2; the loads stay in step order, so the compiler waits for exactly
    // the step it consumes): the weight stream does not pause between flights.
    auto run = [&](Cur c2, auto ring_c) {
        constexpr bool RING = decltype(ring_c)::value;
#pragma unroll
        for (int t = 0; t < FL; ++t) {
            const int b = sb[t];
            if (b != cur_b) {   // wave-uniform; rare (units run block-major)
                const uint8_t* src = img + b * kImgBlock + u * kImgLane;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    a[jj] = __builtin_bit_cast(
                        half8, *reinterpret_cast<const lds_u32x4*>(lds_addr(src + 16 * jj)));
                const float4 rv = *reinterpret_cast<const float4*>(rec + (b * 4 + ip) * kRecBytes);
                rf = rv.x;
                rx = rv.y;
                ry = rv.z;
                cur_b = b;
            }
            uint4 w4;
            if constexpr (B1)
                w4 = uint4{spread_bits(wv[t][0], 0), spread_bits(wv[t][0], 1),
                           spread_bits(wv[t][1], 0), spread_bits(wv[t][1], 1)};
            else
                w4 = wv[t];
            const auto p01 = __builtin_amdgcn_permlane32_swap(w4.x, w4.y, false, false);
            const auto p23 = __builtin_amdgcn_permlane32_swap(w4.z, w4.w, false, false);
            float4v dx = float4v{0.0f, 0.0f, 0.0f, 0.0f};
            float4v dy = float4v{0.0f, 0.0f, 0.0f, 0.0f};
            dx = mac_eword(p01[0], a[0], a[1], dx);
            dy = mac_eword(p01[1], a[2], a[3], dy);
            dx = mac_eword(p23[0], a[4], a[5], dx);
            dy = mac_eword(p23[1], a[6], a[7], dy);
            const float part = (h2f(sv[t] & 0xFFFFu) * (pick(dx, ip) + rx) +
                                h2f(sv[t] >> 16) * (pick(dy, ip) + ry)) *
                               rf;
            if (diag) red[red_lane + sro[t]] = part;
            if constexpr (RING) {
                load_step(t, c2);
                __builtin_amdgcn_sched_barrier(0);
                c2 = cur_next(c2);
            }
        }
    };
    using Plain = std::false_type;
    using Ring = std::true_type;
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
    // images was measured slower).  Only the lanes that hold activations load
    // them (loads that return zeros would still take the address units' time
    // ahead of the weight loads), and no wave waits for them before its weight
    // loads go out.
    uint4 xraw[4];
    if constexpr (ROT) {
        // wave w rotates blocks w and w + kWaves (nb <= 32), stage 1 on the
        // matrix cores
        rot::In rin[2];
        rot::load(x, signs, nb, wave, lane, rin[0]);
        rot::load(x, signs, nb, wave + kWaves, lane, rin[1]);
        set_chunk(0);
        issue(first, Zero{}, Head{});
        __builtin_amdgcn_sched_barrier(0);   // the rotation stays below those weight loads
        rot::half8v hb[2];
        rot::h_operand(lane, hb);
        if (wave < nb) rot::run(rin[0], hb, lane, xrot + wave * kBlock);
        if (wave + kWaves < nb) rot::run(rin[1], hb, lane, xrot + (wave + kWaves) * kBlock);
        lds_barrier();
        if (blockIdx.x == 0)
            for (int i = tid; i < nb * 128; i += kThreads)
                reinterpret_cast<uint4*>(x_rot)[i] = reinterpret_cast<const uint4*>(xrot)[i];
        load_x_lds(xrot, nb, tid, xraw);
        if (wave * 64 < nb * 32) build_pass(xraw, nb, tid, img, rec);
    } else {
        load_x(x, nb, tid, xraw);
        set_chunk(0);
        issue(first, Zero{}, Head{});
        __builtin_amdgcn_sched_barrier(0);   // the image build stays below those weight loads
        if (wave * 64 < nb * 32) build_pass(xraw, nb, tid, img, rec);   // nb * 32 <= kThreads
    }
    lds_barrier();
    if (FL <= kRingMaxFL && flights > 1 && flights <= kRingFlights + 1) {
        // the first chunk's flights as a ring (unrolled: a loop would carry
        // loads in flight across its back edge, and the compiler would then
        // wait for all of them at the top of every flight); nothing else is
        // in flight when it starts (a real wait instruction, which the
        // compiler's wait placement takes into account)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vector memory count 0
        issue(first, Head{}, All{});
        Cur c = first;
#pragma unroll
        for (int f = 0; f < kRingFlights; ++f)
            if (f + 1 < flights) {
                const Cur n = advance(c);
                run(n, Ring{});
                c = n;
            }
        run(c, Plain{});
    } else {
        issue(first, Head{}, All{});
        run(first, Plain{});
        Cur c = first;
        for (int f = 1; f < flights; ++f) {
            c = advance(c);
            issue(c, Zero{}, All{});
            run(c, Plain{});
        }
    }
    finish_chunk();
    for (int c0 = rows_per_chunk; c0 < rows; c0 += rows_per_chunk) {
        set_chunk(c0);
        Cur c = first;
        for (int f = 0; f < flights; ++f) {
            issue(c, Zero{}, All{});
            run(c, Plain{});
            c = advance(c);
        }
        finish_chunk();
    }
}

template <int FL, bool ROT, bool B1>
hipError_t launch_fl(unsigned grid, size_t lds, const uint8_t* packed, const uint16_t* scales,
                     const uint16_t* x, const int8_t* signs, uint16_t* x_rot, int64_t n,
                     int64_t k, int rpc, void* y, int y_f16, hipStream_t stream) {
    const int base = int(n / grid), rem = int(n % grid);
    const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(gemv_m1_slot2_kernel<FL, ROT, B1>), int(kLdsLimit));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_m1_slot2_kernel<FL, ROT, B1>), dim3(grid), dim3(kThreads), lds, stream,
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
    const int64_t grid = n < cu_count() ? n : cu_count();
    const int64_t rows = (n + grid - 1) / grid;                  // largest slice
    int64_t rpc = kMaxSegsPerChunk / nb;
    if (rpc < 1) rpc = 1;
    if (rpc > rows) rpc = rows;
    M1Plan p;
    p.grid = unsigned(grid);
    p.rpc = int(rpc);
    p.steps = int(((rpc + 3) / 4 * nb + kWaves - 1) / kWaves);   // units of 4 rows per wave
    const size_t tail = size_t(nb) * kImgBlock + size_t(nb) * 4 * kRecBytes + size_t(rpc * nb) * 16;
    p.lds = rot ? size_t(nb) * 2048 + tail : tail;   // ROT: the rotated activations first
    return p;
}

template <bool ROT, bool B1>
hipError_t launch_m1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                     const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k, void* y, int y_f16,
                     hipStream_t stream) {
    const M1Plan p = m1_plan(n, k, ROT);
    // up to 8 steps a slot: one flight, every load issued at once; up to
    // 4 flights of kRingMaxFL: a ring; beyond, flights of 8
    if (p.steps > 8 && p.steps <= kRingMaxFL * (kRingFlights + 1))
        return launch_fl<kRingMaxFL, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k,
                                          p.rpc, y, y_f16, stream);
    switch (p.steps) {
        case 1:
            return launch_fl<1, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 2:
            return launch_fl<2, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 3:
            return launch_fl<3, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 4:
            return launch_fl<4, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 5:
            return launch_fl<5, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 6:
            return launch_fl<6, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        case 7:
            return launch_fl<7, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
        default:
            return launch_fl<8, ROT, B1>(p.grid, p.lds, packed, scales, x, signs, x_rot, n, k, p.rpc, y,
                                     y_f16, stream);
    }
}

bool m1_fits(int64_t m, int64_t n, int64_t k, bool rot) {   // both packings
    const int64_t nb = k / kBlock;
    const int64_t grid = n < cu_count() ? n : cu_count();
    const int64_t rows = (n + grid - 1) / grid;
    // one image pass (32 threads per block)
    // and 32-bit buffer offsets
    return m == 1 && nb * 32 <= kThreads && m1_plan(n, k, rot).lds <= kLdsLimit &&
           rows * (k / 4) < (int64_t(1) << 31);
}

}  // namespace

bool gemv_m1_slot2_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, false); }

hipError_t launch_gemv_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    return launch_m1<false, false>(packed, scales, x, nullptr, nullptr, n, k, y, y_f16, stream);
}

bool linear_m1_slot2_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, true); }

hipError_t launch_linear_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                  const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k,
                                  void* y, int y_f16, hipStream_t stream) {
    return launch_m1<true, false>(packed, scales, x, signs, x_rot, n, k, y, y_f16, stream);
}

bool gemv_m1_bit1_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, false); }

hipError_t launch_gemv_m1_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                               int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    return launch_m1<false, true>(packed, scales, x, nullptr, nullptr, n, k, y, y_f16, stream);
}

bool linear_m1_bit1_fits(int64_t m, int64_t n, int64_t k) { return m1_fits(m, n, k, true); }

hipError_t launch_linear_m1_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                 const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k,
                                 void* y, int y_f16, hipStream_t stream) {
    return launch_m1<true, true>(packed, scales, x, signs, x_rot, n, k, y, y_f16, stream);
}

}  // namespace tl
