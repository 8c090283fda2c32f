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
// into LDS by direct global->LDS loads issued ahead of the weights; loads of a
// wave complete in order, so waiting for them does not wait for the weights,
// and the decode table is built while everything is in flight.  The waits are
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
constexpr int flight_max(int nt) { return nt == 1 ? 3 : 2; }
constexpr int kLoadsPerBlock = kSteps + 1; // 16-byte loads per block: codes + scales
constexpr int kMaxWaves = 16;              // waves per workgroup
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
// completion is covered by the explicit wait in wait_barrier.  No register is
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

// Wait until at most N vector-memory loads of this wave are outstanding and
// its LDS writes are done, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void build_lut(uint8_t* lut, int tid, int nthreads) {
    // table rows: consecutive threads write consecutive 16-byte pieces
    for (int c = tid; c < kLutBytes / 16; c += nthreads) {
        const uint32_t b = uint32_t(c) >> 4;
        const uint32_t lo = code_bits(b & 3u) | (code_bits((b >> 2) & 3u) << 16);
        const uint32_t hi = code_bits((b >> 4) & 3u) | (code_bits((b >> 6) & 3u) << 16);
        reinterpret_cast<uint4*>(lut)[c] = uint4{lo, hi, lo, hi};
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

struct Lane {
    const uint8_t* lut;
    uint32_t rep;     // this lane's table copy * 8
    int64_t k;
};

// Decode and multiply one block into acc.  xr points at this lane's
// activations for the block's first step (row of its A role).
template <int NT>
__device__ __forceinline__ void compute_block(const Block& b, const Lane& ln, const uint16_t* xr,
                                              const bool (&a_load)[NT], uint4 (&av)[NT],
                                              float (&acc)[NT][2]) {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const uint32_t s2 = i == 0 ? b.s.x : (i == 1 ? b.s.y : (i == 2 ? b.s.z : b.s.w));
        const float sc0 = __half2float(__ushort_as_half(uint16_t(s2 & 0xFFFFu)));
        const float sc1 = __half2float(__ushort_as_half(uint16_t(s2 >> 16)));
        float4v d[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) d[p] = float4v{0.f, 0.f, 0.f, 0.f};
        const uint32_t wd[4] = {b.w[i].x, b.w[i].y, b.w[i].z, b.w[i].w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t dw = wd[t >> 1];
            const uint32_t a0 = (t & 1) ? lut_addr<2>(ln.rep, dw) : lut_addr<0>(ln.rep, dw);
            const uint32_t a1 = (t & 1) ? lut_addr<3>(ln.rep, dw) : lut_addr<1>(ln.rep, dw);
            const uint2 e0 = *reinterpret_cast<const uint2*>(ln.lut + a0);
            const uint2 e1 = *reinterpret_cast<const uint2*>(ln.lut + a1);
            const half8 bv = __builtin_bit_cast(half8, uint4{e0.x, e0.y, e1.x, e1.y});
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                // activations x[tok][256 s + 64 q + 8 t .. + 7] of this lane's A role
                if (a_load[p])
                    av[p] = *reinterpret_cast<const uint4*>(xr + 8 * p * ln.k + 256 * i + 8 * t);
                d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(half8, av[p]), bv, d[p], 0, 0, 0);
            }
        }
        // D row 4q + r = token 2q + r/2 of the pass, group parity r & 1
#pragma unroll
        for (int p = 0; p < NT; ++p) {
            acc[p][0] += sc0 * d[p][0] + sc1 * d[p][1];
            acc[p][1] += sc0 * d[p][2] + sc1 * d[p][3];
        }
    }
}

// NR consecutive blocks of this wave's tile: all loads first, then the
// blocks in order.  The first flight of the kernel also builds the table and
// holds the workgroup barrier that publishes the table and the activations:
// at that point only the NR blocks were issued after the activation copies.
template <int NR, int NT, bool FIRST>
__device__ __forceinline__ void flight(const uint8_t* wb, const uint16_t* sb, const uint16_t* xr,
                                       const Lane& ln, uint8_t* lut, int tid, int nthreads,
                                       const bool (&a_load)[NT], uint4 (&av)[NT],
                                       float (&acc)[NT][2]) {
    Block b[NR > 0 ? NR : 1];
#pragma unroll
    for (int i = 0; i < NR; ++i) load_block(b[i], wb + 256 * i, sb + 8 * i);
    if (FIRST) {
        build_lut(lut, tid, nthreads);
        wait_barrier<kLoadsPerBlock * NR>();
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) compute_block<NT>(b[i], ln, xr + 1024 * i, a_load, av, acc);
}

template <int NT, bool FIRST>
__device__ __forceinline__ void flight_n(int nr, const uint8_t* wb, const uint16_t* sb,
                                         const uint16_t* xr, const Lane& ln, uint8_t* lut, int tid,
                                         int nthreads, const bool (&a_load)[NT], uint4 (&av)[NT],
                                         float (&acc)[NT][2]) {
    if (flight_max(NT) >= 3 && nr >= 3)
        flight<(flight_max(NT) >= 3 ? 3 : 2), NT, FIRST>(wb, sb, xr, ln, lut, tid, nthreads,
                                                         a_load, av, acc);
    else if (nr >= 2)
        flight<2, NT, FIRST>(wb, sb, xr, ln, lut, tid, nthreads, a_load, av, acc);
    else if (nr == 1)
        flight<1, NT, FIRST>(wb, sb, xr, ln, lut, tid, nthreads, a_load, av, acc);
    else if (FIRST)
        flight<0, NT, FIRST>(wb, sb, xr, ln, lut, tid, nthreads, a_load, av, acc);
}

template <int NT, bool XLDS>
__global__ __launch_bounds__(1024) void gemv_slot2_kernel(
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

    // activations -> LDS, 1 KB per wave instruction, issued before any weight
    // load; surplus instructions repeat the last piece (same bytes, same place)
    if (XLDS) {
        const int pieces = int(int64_t(m) * k / 512);   // M*K is a multiple of 1024
        const int per_wave = (pieces + nwaves - 1) / nwaves;
        const uint32_t xs_off =
            uint32_t(uintptr_t((__attribute__((address_space(3))) uint16_t*)(xs)));
        for (int c = 0; c < per_wave; ++c) {
            int idx = wave + c * nwaves;
            idx = idx < pieces ? idx : pieces - 1;
            dma_1k(xs_off + uint32_t(idx) * 1024u, x + int64_t(idx) * 512 + lane * 8);
        }
    }

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

    const Lane ln{lut, uint32_t(lane & 31) * 8u, k};
    // A-operand role of this lane: row j of A = token j/2 of the pass, parity j&1
    const int a_tok = j >> 1, a_par = j & 1;
    const bool a_live = a_par == (q >> 1);
    bool a_load[NT];
    float acc[NT][2];
    uint4 av[NT];   // lanes without activations keep zeros for the whole kernel
#pragma unroll
    for (int p = 0; p < NT; ++p) {
        acc[p][0] = acc[p][1] = 0.0f;
        a_load[p] = a_live && (8 * p + a_tok) < m;
        av[p] = uint4{0, 0, 0, 0};
    }
    // activations of this lane's A role: LDS copy or global memory
    const int64_t xoff = int64_t(a_tok) * k + 64 * q + kBlock * b0;
    const uint16_t* xr = XLDS ? static_cast<const uint16_t*>(xs + xoff) : x + xoff;

    int64_t tile = tile_slot;
    int64_t row = r0 + 16 * tile + j;
    bool row_ok = tile < tiles_here && row < r1;
    // rows past the slice re-read row r0 (a valid row) and are never written
    const int64_t lrow = row_ok ? row : r0;
    const uint8_t* wb = packed + lrow * row_bytes + 16 * q + 256 * b0;
    const uint16_t* sb = scales + lrow * groups + 8 * b0;
    const int nb = tile < tiles_here ? nb_tile : 0;

    constexpr int kFlight = flight_max(NT);
    int f = nb < kFlight ? nb : kFlight;
    flight_n<NT, true>(f, wb, sb, xr, ln, lut, tid, nthreads, a_load, av, acc);
    for (;;) {   // tiles of this wave (a single one unless ksplit == 1)
        for (; f < nb; f += kFlight)
            flight_n<NT, false>(nb - f, wb + 256 * f, sb + 8 * f, xr + kBlock * f, ln, lut, tid,
                                nthreads, a_load, av, acc);
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
        f = 0;
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

struct Plan {
    int64_t grid;
    int ksplit;
    int waves;
};

// one workgroup per CU, each with an equal share of the rows; the waves of a
// workgroup split K when the share is at most 16 tiles
Plan make_plan(int64_t n) {
    Plan p;
    const int64_t tiles = (n + 15) / 16;
    p.grid = tiles < num_cus() ? tiles : num_cus();
    const int64_t rows_per_wg = (n + p.grid - 1) / p.grid;
    const int64_t tiles_per_wg = (rows_per_wg + 15) / 16;
    if (tiles_per_wg >= kMaxWaves) {
        p.ksplit = 1;
        p.waves = kMaxWaves;
    } else {
        p.ksplit = int(kMaxWaves / tiles_per_wg);
        p.waves = int(tiles_per_wg) * p.ksplit;
    }
    return p;
}

template <int NT, bool XLDS>
hipError_t launch_one(const Plan& plan, const uint8_t* packed, const uint16_t* scales,
                      const uint16_t* x, int mt, int64_t n, int64_t k, void* y, int y_f16,
                      hipStream_t stream) {
    static bool attr_set = false;
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(gemv_slot2_kernel<NT, XLDS>),
            hipFuncAttributeMaxDynamicSharedMemorySize, int(kLdsLimit));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    size_t lds = size_t(kLutBytes) + size_t(plan.waves) * NT * 2 * 64 * 4 +
                 (XLDS ? size_t(mt) * size_t(k) * 2 : 0);
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
    const Plan plan = make_plan(n);
    // activations go to LDS when they fit beside the table and the reduction buffer
    const int64_t x_lds_budget = int64_t(kLdsLimit) - kLutBytes - kMaxWaves * 2 * 2 * 64 * 4;
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mt = int(m - m0 < 16 ? m - m0 : 16);
        const uint16_t* xs = x + m0 * k;
        void* ys = static_cast<uint8_t*>(y) + m0 * n * y_elem;
        const bool fits = int64_t(mt) * k * 2 <= x_lds_budget;
        hipError_t e;
        if (mt <= 8)
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
