// Decode GEMV for the 2-bit-slot packing on fp16 matrix cores.
//
//   y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[m, k]
//
// Ternary multiply-accumulate is additions and subtractions (page "Ternary
// Bonsai 2 27B", section "Что такое тернарная модель"); here the codes are
// expanded to binary16 {-1, 0, +1} (exact) and the additions run on the
// matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation), while each
// 128-group is scaled once by its binary16 scale in an fp32 epilogue (page
// "A 27-billion model that fits in 8.6 GB", paragraph 2).
//
// Roles: the MFMA A operand holds activations (rows = tokens), B holds weights
// (columns = 16 weight rows of a tile).  One workgroup of up to 16 waves runs
// per CU and owns an equal slice of the rows (so every CU streams the same
// number of bytes); the slice is cut into 16-row tiles (the last one may be
// partial) and the waves split the 1024-blocks of each tile's K into ksplit
// ranges, reduced through LDS in a fixed order (bitwise deterministic).
//
// Memory pipeline.  A decode GEMV touches every weight byte once, and at the
// model's shapes a CU's share is only a few blocks per wave, so each wave
// requests all the blocks it owns (up to kFlight at a time, held in
// registers) before it waits for any of them.  The activations are copied
// into LDS by direct global->LDS loads, and the decode table is built, before
// the weight stream starts (see the prologue).  The waits are
// explicit counts on straight-line code (one instantiation per number of
// blocks in flight), so no wait covers a load that is not yet needed.
//
// Chunk step: 64 bytes (two 128-groups) of each of the 16 rows: lane
// (j = lane % 16, q = lane / 16) holds the 16 bytes [16q, 16q + 16) of row j,
// i.e. half of group 2s + q/2.  MFMA t (t = 0..7) takes bytes 2t and 2t + 1 of
// every lane's chunk, so its 32 K-slots come from two groups; A rows are
// split by group parity (row 2*token + p only carries activations of the
// lanes whose bytes lie in group 2s + p), which keeps the two groups apart in
// D and lets the epilogue apply each group's scale.  Up to 8 tokens per pass;
// NT passes share every decoded weight tile.
//
// Decode table (LDS): entry b holds the four binary16 codes of packed byte b;
// 32 copies staggered by 8 bytes fill a 256-byte row, so the 32 lanes that a
// 64-bit LDS read serves per cycle hit 64 distinct banks whatever bytes they
// decode, and one v_perm_b32 builds the address b * 256 + copy * 8.  Valid
// bytes are below 171 (the top slot holds a digit <= 2), so 171 rows suffice.
#include <hip/hip_fp16.h>

#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kLutRows = 171;              // bytes 0..170 cover every valid code pattern
constexpr int kLutBytes = kLutRows * 256;
constexpr int kSteps = 4;                  // 64-byte chunk steps per 1024-block
// blocks a wave keeps in flight (registers: 20 VGPRs per block)
constexpr int flight_max(int nt) { return nt == 1 ? 2 : 2; }
// waves per workgroup: 16 (128 VGPRs each) for one pass, 8 (256 VGPRs each)
// for two passes, whose operands need the larger register budget
constexpr int max_waves(int nt) { return nt == 1 ? 16 : 8; }
constexpr size_t kLdsLimit = 160 * 1024;

__device__ __forceinline__ uint32_t code_bits(uint32_t d) {
    // digit -> binary16 bits of (d - 1); digit 3 never occurs in valid data
    return d == 0u ? 0xBC00u : (d == 2u ? 0x3C00u : 0u);
}

struct Block {
    uint4 w[kSteps];  // this lane's 16 bytes of each chunk step
    uint4 s;          // the block's 8 scales: group 2i + p of step i is half 2i + p
};

// The weight pointers carry no __restrict__: that keeps these loads on their
// side of the asm barrier below (memory clobber) instead of sinking them
// towards their first use.
__device__ __forceinline__ void load_block(Block& b, const uint8_t* wb, const uint16_t* sb) {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) b.w[i] = *reinterpret_cast<const uint4*>(wb + 64 * i);
    b.s = *reinterpret_cast<const uint4*>(sb);
}

// Copy 1 KB (16 bytes per lane) from global memory straight into LDS at the
// wave-uniform byte offset lds_off.  Issued from asm so that the compiler does
// not track it (it would otherwise wait for every load before any LDS read);
// completion is covered by the explicit wait in vm_lds_barrier.  No register is
// written, so nothing is left in flight that the compiler could reuse.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved, and set here on purpose
__device__ __forceinline__ void dma_1k(uint32_t lds_off, const void* src) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_off), "v"(src)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait for every load and LDS write of this wave (the activation copies are
// tracked by no compiler-inserted wait), then the workgroup barrier.
__device__ __forceinline__ void vm_lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void build_lut(uint8_t* lut, int tid, int nthreads) {
    // Thread t fills row b = t / 4 (16 pieces of 16 bytes, two copies each):
    // it decodes byte b once and writes pieces r, r + 4, r + 8 and r + 12
    // (r = t % 4), starting with piece (r + 4 b) % 16, so the 16 lanes that an
    // LDS write serves together hit 16 distinct 16-byte bank groups.
    for (int t = tid; t < 4 * kLutRows; t += nthreads) {
        const uint32_t b = uint32_t(t) >> 2, r = uint32_t(t) & 3u;
        const uint32_t lo = code_bits(b & 3u) | (code_bits((b >> 2) & 3u) << 16);
        const uint32_t hi = code_bits((b >> 4) & 3u) | (code_bits((b >> 6) & 3u) << 16);
        const uint4 e = uint4{lo, hi, lo, hi};
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i)
            reinterpret_cast<uint4*>(lut)[b * 16 + ((r + 4 * (b + i)) & 15u)] = e;
    }
}

__device__ __forceinline__ void store_y(void* y, int y_f16, int64_t o, float v) {
    if (y_f16)
        reinterpret_cast<__half*>(y)[o] = __float2half_rn(v);
    else
        reinterpret_cast<float*>(y)[o] = v;
}

// LDS byte address of the table entry for byte `sel_byte` of w, in this
// lane's copy: bits 0-7 = copy * 8 (from rep), bits 8-15 = the byte, rest 0.
template <int SEL_BYTE>
__device__ __forceinline__ uint32_t lut_addr(uint32_t rep, uint32_t w) {
    // v_perm_b32: selector bytes 0-3 pick bytes of the second source, 4-7
    // bytes of the first, 0x0c gives zero.
    return __builtin_amdgcn_perm(rep, w, 0x0c0c0004u | (uint32_t(SEL_BYTE) << 8));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// Where a lane's A operand (activations) comes from.  Offsets are byte
// offsets from the start of the wave's K range, the same for every lane.
template <int NT, bool XLDS>
struct XSrc;

// LDS copy: per pass, the LDS byte address of the lane's activations at the
// start of its K range, or of a 128-byte zero pad for lanes that carry none;
// the mask keeps the pad address fixed, so no lane branches or zero-fills.
template <int NT>
struct XSrc<NT, true> {
    uint32_t base[NT];
    uint32_t mask[NT];
    __device__ __forceinline__ uint4 get(int p, uint32_t off, int t) const {
        return __builtin_bit_cast(
            uint4, *reinterpret_cast<lds_u32x4*>(base[p] + (mask[p] & off) + 16u * uint32_t(t)));
    }
};

// Global memory (activations too large for LDS): lanes that carry none read
// nothing and take zeros.
template <int NT>
struct XSrc<NT, false> {
    const uint8_t* ptr[NT];
    bool live[NT];
    __device__ __forceinline__ uint4 get(int p, uint32_t off, int t) const {
        return live[p] ? *reinterpret_cast<const uint4*>(ptr[p] + off + 16 * t)
                       : uint4{0, 0, 0, 0};
    }
};

// MFMAs per batch of operand reads: the whole step for one pass, half of it
// for two
template <int NT>
constexpr int batch() { return NT == 1 ? 8 : 4; }

// Decode and multiply one block into acc; off = byte offset of the block in
// the wave's K range.  Operand reads (activation pieces and table entries) are
// issued in batches ahead of their MFMAs, so the LDS latency is paid once per
// batch rather than per MFMA.  The table sits at LDS address 0, so the
// v_perm_b32 result is the entry's address.
template <int NT, bool XLDS>
__device__ __forceinline__ void compute_block(const Block& b, uint32_t rep, const XSrc<NT, XLDS>& xs,
                                              uint32_t off, float (&acc)[NT][2]) {
    constexpr int TB = batch<NT>();
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const uint32_t wd[4] = {b.w[i].x, b.w[i].y, b.w[i].z, b.w[i].w};
        float4v d[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) d[p] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t0 = 0; t0 < 8; t0 += TB) {
            // activations x[tok][256 s + 64 q + 8 t .. + 7] of this lane's A role
            uint4 av[NT][TB];
#pragma unroll
            for (int p = 0; p < NT; ++p)
#pragma unroll
                for (int t = 0; t < TB; ++t) av[p][t] = xs.get(p, off + 512u * i, t0 + t);
            uint2 e[2 * TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const int tt = t0 + t;
                const uint32_t dw = wd[tt >> 1];
                const uint32_t a0 = (tt & 1) ? lut_addr<2>(rep, dw) : lut_addr<0>(rep, dw);
                const uint32_t a1 = (tt & 1) ? lut_addr<3>(rep, dw) : lut_addr<1>(rep, dw);
                e[2 * t] = __builtin_bit_cast(uint2, *reinterpret_cast<lds_u32x2*>(a0));
                e[2 * t + 1] = __builtin_bit_cast(uint2, *reinterpret_cast<lds_u32x2*>(a1));
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const half8 bv = __builtin_bit_cast(
                    half8, uint4{e[2 * t].x, e[2 * t].y, e[2 * t + 1].x, e[2 * t + 1].y});
#pragma unroll
                for (int p = 0; p < NT; ++p)
                    d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(half8, av[p][t]), bv, d[p], 0, 0, 0);
            }
        }
        // D row 4q + r = token 2q + r/2 of the pass, group parity r & 1
        const uint32_t s2 = i == 0 ? b.s.x : (i == 1 ? b.s.y : (i == 2 ? b.s.z : b.s.w));
        const float sc0 = __half2float(__ushort_as_half(uint16_t(s2 & 0xFFFFu)));
        const float sc1 = __half2float(__ushort_as_half(uint16_t(s2 >> 16)));
#pragma unroll
        for (int p = 0; p < NT; ++p) {
            acc[p][0] += sc0 * d[p][0] + sc1 * d[p][1];
            acc[p][1] += sc0 * d[p][2] + sc1 * d[p][3];
        }
    }
}

// NR consecutive blocks of this wave's tile: all loads first, then the
// blocks in order.
template <int NR, int NT, bool XLDS>
__device__ __forceinline__ void flight(const uint8_t* wb, const uint16_t* sb, uint32_t rep,
                                       const XSrc<NT, XLDS>& xs, uint32_t off,
                                       float (&acc)[NT][2]) {
    Block b[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) load_block(b[i], wb + 256 * i, sb + 8 * i);
#pragma unroll
    for (int i = 0; i < NR; ++i)
        compute_block<NT, XLDS>(b[i], rep, xs, off + 2048u * i, acc);
}

template <int NT, bool XLDS>
__device__ __forceinline__ void flight_n(int nr, const uint8_t* wb, const uint16_t* sb,
                                         uint32_t rep, const XSrc<NT, XLDS>& xs, uint32_t off,
                                         float (&acc)[NT][2]) {
    constexpr int kTop = flight_max(NT) >= 3 ? 3 : 2;
    if (kTop == 3 && nr >= 3)
        flight<kTop, NT, XLDS>(wb, sb, rep, xs, off, acc);
    else if (nr >= 2)
        flight<2, NT, XLDS>(wb, sb, rep, xs, off, acc);
    else if (nr == 1)
        flight<1, NT, XLDS>(wb, sb, rep, xs, off, acc);
}

template <int NT, bool XLDS>
__global__ __launch_bounds__(64 * max_waves(NT)) void gemv_slot2_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int m, int64_t n, int64_t k,
    int ksplit, void* __restrict__ y, int y_f16) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* lut = smem;
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    float* red = reinterpret_cast<float*>(smem + kLutBytes);       // [wave][NT][2][64]
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem + kLutBytes + nwaves * NT * 2 * 64 * 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;          // weight row in the tile (B column) / A row
    const int q = lane >> 4;          // 16-byte piece of the lane inside a chunk step

    // this workgroup's rows, and this wave's tile and block range
    const int64_t r0 = int64_t(blockIdx.x) * n / gridDim.x;
    const int64_t r1 = int64_t(blockIdx.x + 1) * n / gridDim.x;
    const int tile_slot = wave / ksplit;
    const int ks = wave - tile_slot * ksplit;
    const int tile_stride = nwaves / ksplit;          // > 1 tile per wave only when ksplit == 1
    const int64_t tiles_here = (r1 - r0 + 15) / 16;
    const int64_t row_bytes = k / 4;
    const int64_t groups = k / kGroup;
    const int64_t blocks = k / kBlock;
    const int64_t b0 = blocks * ks / ksplit;
    const int nb_tile = int(blocks * (ks + 1) / ksplit - b0);
    const int nb = tile_slot < tiles_here ? nb_tile : 0;

    // Prologue: the activations -> LDS (1 KB per wave instruction, spread over
    // the waves) and the decode table, published by one barrier before any
    // weight load is issued.  The activations are read by every CU; requested
    // while the weight stream is in flight they would queue behind it in the
    // shared memory queues and hold the first MFMA back until most weights
    // had arrived.
    const uint32_t xs_lds = uint32_t(uintptr_t((__attribute__((address_space(3))) uint16_t*)(xs)));
    const uint32_t zero_lds = xs_lds + uint32_t(m) * uint32_t(k) * 2u;   // 128-byte zero pad
    if (XLDS) {
        const int pieces = int(int64_t(m) * k / 512);   // M*K is a multiple of 1024
        for (int c = wave; c < pieces; c += nwaves)
            dma_1k(xs_lds + uint32_t(c) * 1024u, x + int64_t(c) * 512 + lane * 8);
        if (tid < 8)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(zero_lds + 16u * tid) =
                u32x4{0, 0, 0, 0};
    }
    build_lut(lut, tid, nthreads);
    vm_lds_barrier();

    const uint32_t rep = uint32_t(lane & 31) * 8u;   // this lane's table copy * 8
    // A-operand role of this lane: row j of A = token j/2 of the pass, parity j&1
    const int a_tok = j >> 1, a_par = j & 1;
    const bool a_live = a_par == (q >> 1);
    float acc[NT][2];
    XSrc<NT, XLDS> xsrc;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
        acc[p][0] = acc[p][1] = 0.0f;
        const bool live = a_live && (8 * p + a_tok) < m;
        const int64_t xoff = int64_t(8 * p + a_tok) * k + 64 * q + kBlock * b0;   // halves
        if constexpr (XLDS) {
            xsrc.base[p] = live ? xs_lds + uint32_t(xoff) * 2u : zero_lds;
            xsrc.mask[p] = live ? ~0u : 0u;
        } else {
            xsrc.ptr[p] = reinterpret_cast<const uint8_t*>(x + (live ? xoff : 0));
            xsrc.live[p] = live;
        }
    }

    int64_t tile = tile_slot;
    int64_t row = r0 + 16 * tile + j;
    bool row_ok = tile < tiles_here && row < r1;
    // rows past the slice re-read row r0 (a valid row) and are never written
    const int64_t lrow = row_ok ? row : r0;
    const uint8_t* wb = packed + lrow * row_bytes + 16 * q + 256 * b0;
    const uint16_t* sb = scales + lrow * groups + 8 * b0;

    constexpr int kFlight = flight_max(NT);
    for (;;) {   // tiles of this wave (a single one unless ksplit == 1)
        for (int f = 0; f < nb; f += kFlight)
            flight_n<NT, XLDS>(nb - f, wb + 256 * f, sb + 8 * f, rep, xsrc, 2048u * uint32_t(f),
                               acc);
        tile += tile_stride;
        if (ksplit > 1 || tile >= tiles_here) break;
        // whole-K tiles: write this one out and start the next
        if (row_ok) {
#pragma unroll
            for (int p = 0; p < NT; ++p)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int tok = 8 * p + 2 * q + h;
                    if (tok < m) store_y(y, y_f16, int64_t(tok) * n + row, acc[p][h]);
                }
        }
#pragma unroll
        for (int p = 0; p < NT; ++p) acc[p][0] = acc[p][1] = 0.0f;
        row = r0 + 16 * tile + j;
        row_ok = row < r1;
        const int64_t nrow = row_ok ? row : r0;
        wb = packed + nrow * row_bytes + 16 * q;
        sb = scales + nrow * groups;
    }

#pragma unroll
    for (int p = 0; p < NT; ++p) {
        red[((wave * NT + p) * 2 + 0) * 64 + lane] = acc[p][0];
        red[((wave * NT + p) * 2 + 1) * 64 + lane] = acc[p][1];
    }
    __syncthreads();
    if (ks == 0 && row_ok) {
#pragma unroll
        for (int p = 0; p < NT; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tok = 8 * p + 2 * q + h;
                if (tok < m) {
                    float v = red[((wave * NT + p) * 2 + h) * 64 + lane];
                    for (int w2 = 1; w2 < ksplit; ++w2)
                        v += red[(((wave + w2) * NT + p) * 2 + h) * 64 + lane];
                    store_y(y, y_f16, int64_t(tok) * n + row, v);
                }
            }
    }
}

struct Plan {
    int64_t grid;
    int ksplit;
    int waves;
};

// one workgroup per CU, each with an equal share of the rows; the waves of a
// workgroup split K when the share is at most max_waves tiles
Plan make_plan(int64_t n, int max_w) {
    Plan p;
    const int64_t tiles = (n + 15) / 16;
    p.grid = tiles < cu_count() ? tiles : cu_count();
    const int64_t rows_per_wg = (n + p.grid - 1) / p.grid;
    const int64_t tiles_per_wg = (rows_per_wg + 15) / 16;
    if (tiles_per_wg >= max_w) {
        p.ksplit = 1;
        p.waves = max_w;
    } else {
        p.ksplit = int(max_w / tiles_per_wg);
        p.waves = int(tiles_per_wg) * p.ksplit;
    }
    return p;
}

template <int NT, bool XLDS>
hipError_t launch_one(const Plan& plan, const uint8_t* packed, const uint16_t* scales,
                      const uint16_t* x, int mt, int64_t n, int64_t k, void* y, int y_f16,
                      hipStream_t stream) {
    const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(gemv_slot2_kernel<NT, XLDS>), int(kLdsLimit));
    if (e != hipSuccess) return e;
    size_t lds = size_t(kLutBytes) + size_t(plan.waves) * NT * 2 * 64 * 4 +
                 (XLDS ? size_t(mt) * size_t(k) * 2 + 128 : 0);
    // ask for more than half of the CU's LDS so that two workgroups never share a CU
    if (lds < kLdsLimit / 2 + 1024) lds = kLdsLimit / 2 + 1024;
    hipLaunchKernelGGL((gemv_slot2_kernel<NT, XLDS>), dim3(unsigned(plan.grid)),
                       dim3(64 * plan.waves), lds, stream, packed, scales, x, mt, n, k,
                       plan.ksplit, y, y_f16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream) {
    const int64_t y_elem = y_f16 ? 2 : 4;
    // up to 16 tokens per launch: one pass of 8, or two passes sharing the decode
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mt = int(m - m0 < 16 ? m - m0 : 16);
        const int nt = mt <= 8 ? 1 : 2;
        const Plan plan = make_plan(n, max_waves(nt));
        const uint16_t* xs = x + m0 * k;
        void* ys = static_cast<uint8_t*>(y) + m0 * n * y_elem;
        // activations go to LDS (with a 128-byte zero pad) when they fit beside
        // the table and the reduction buffer
        const int64_t x_lds_budget =
            int64_t(kLdsLimit) - kLutBytes - int64_t(plan.waves) * nt * 2 * 64 * 4;
        const bool fits = int64_t(mt) * k * 2 + 128 <= x_lds_budget;
        hipError_t e;
        if (nt == 1)
            e = fits ? launch_one<1, true>(plan, packed, scales, xs, mt, n, k, ys, y_f16, stream)
                     : launch_one<1, false>(plan, packed, scales, xs, mt, n, k, ys, y_f16, stream);
        else
            e = fits ? launch_one<2, true>(plan, packed, scales, xs, mt, n, k, ys, y_f16, stream)
                     : launch_one<2, false>(plan, packed, scales, xs, mt, n, k, ys, y_f16, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tl
