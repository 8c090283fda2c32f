// Decode GEMV for the dense trit packing on fp16 matrix cores.
//
//   y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[m, k]
//
// The packing stores five codes per byte as base-3 digits d = code + 1, 26
// bytes per 128-group (25 full bytes and a tail byte with three codes); this
// is how the dense trit format reaches its density (page "A 27-billion model
// that fits in 8.6 GB", paragraphs 2 and 5; the byte layout itself is this
// library's, defined in include/tl.h).  Codes are expanded to binary16
// {-1, 0, +1} (exact) and multiplied on the matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation); each group is scaled once by
// its binary16 scale in an fp32 epilogue (same page, paragraph 2).
//
// Work split (as for the 2-bit-slot kernel): one workgroup per CU owns an
// equal share of the rows in 16-row tiles; the waves split each tile's
// 1024-blocks into ksplit ranges, reduced through LDS in a fixed order
// (bitwise deterministic); the activations and the decode table are staged in
// LDS before the weight stream starts, and each wave requests all blocks it
// owns (up to a flight) before it waits for any.
//
// Block layout.  A 1024-block of a row is 8 groups = 208 bytes.  Lane
// (j = lane % 16, q = lane / 16) holds bytes [52q, 52q + 52) of the block of
// row j: exactly groups 2q and 2q + 1 (one 4-byte-aligned 52-byte piece, read
// as three 16-byte loads and one 4-byte load).  The 128 codes of a group,
// read in order, form 16 windows of 8 codes, and window w of group 2q + h is
// this lane's share of MFMA (h, w): 32 K-slots, 8 from each of the four
// lanes of the row, all real codes (the tail byte's two pad digits are never
// read).  A row 4*token + c of the A operand carries the activations of lane
// group c only, so D row (token, c) holds group 2c + h alone and the
// epilogue applies its scale.  Up to 4 tokens per pass, NT passes per launch.
//
// Decode table (at LDS address 0): entry v holds the five binary16 codes of
// byte value v in halves 0..4 (halves 5..7 zero); 16 copies 16 bytes apart
// fill a 256-byte row, so the 16 lanes that a 128-bit LDS read serves per
// cycle hit distinct banks whatever bytes they decode, and one v_perm_b32
// builds the address v * 256 + copy * 16.  Rows 243..255 (no valid byte)
// decode to zeros.  A window's four code pairs are whole or spliced dwords of
// consecutive entries; the splice positions are fixed per window, so each is
// one v_perm_b32 with a constant selector.
#include <hip/hip_fp16.h>

#include "rotate_lds.h"
#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

constexpr int kLutBytes = 256 * 256;       // 256 rows of 16 copies x 16 bytes
constexpr int kBlockBytes = 208;           // 8 groups x 26 bytes
constexpr int kPieceBytes = 52;            // one lane's two groups
constexpr int64_t kLdsLimit = 160 * 1024;

// waves per workgroup: 16 (128 VGPRs each) for one pass, 8 (256 VGPRs) for
// more passes
template <int NT>
constexpr int waves() { return NT == 1 ? 16 : 8; }
// blocks a wave keeps in flight (17 VGPRs each)
template <int NT>
constexpr int flight_max() { return NT == 1 ? 2 : (NT == 2 ? 2 : 1); }

struct Block {
    uint4 w[3];       // bytes 0..47 of the lane's 52-byte piece
    uint32_t w3;      // bytes 48..51
    uint4 s;          // the block's 8 scales of the lane's row
};

// The pointers carry no __restrict__ so that the loads stay where they are
// written (issued before the first wait) instead of sinking to their use.
__device__ __forceinline__ void load_block(Block& b, const uint8_t* wb, const uint16_t* sb) {
#pragma unroll
    for (int i = 0; i < 3; ++i) b.w[i] = *reinterpret_cast<const uint4*>(wb + 16 * i);
    b.w3 = *reinterpret_cast<const uint32_t*>(wb + 48);
    b.s = *reinterpret_cast<const uint4*>(sb);
}

// Copy 1 KB (16 bytes per lane) from global memory straight into LDS at the
// wave-uniform byte offset lds_off (see the 2-bit-slot kernel).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
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

__device__ __forceinline__ uint32_t code_bits(uint32_t d) {
    // digit -> binary16 bits of (d - 1)
    return d == 0u ? 0xBC00u : (d == 2u ? 0x3C00u : 0u);
}

__device__ __forceinline__ void build_lut(uint8_t* lut, int tid, int nthreads) {
    // Thread t fills row v = t / 4: it decodes byte value v once and writes
    // copies r, r + 4, r + 8 and r + 12 (r = t % 4), starting with copy
    // (r + 4 v) % 16, so the 16 lanes that an LDS write serves together hit 16
    // distinct 16-byte bank groups.
    for (int t = tid; t < 1024; t += nthreads) {
        const uint32_t v = uint32_t(t) >> 2, r = uint32_t(t) & 3u;
        uint32_t h[5] = {0, 0, 0, 0, 0};
        if (v < 243) {
            uint32_t rem = v;
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                h[i] = code_bits(rem % 3u);
                rem /= 3u;
            }
        }
        const uint4 e = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u};
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i)
            reinterpret_cast<uint4*>(lut)[v * 16 + ((r + 4 * (v + i)) & 15u)] = e;
    }
}

// byte i (0..51) of the lane's piece
__device__ __forceinline__ uint32_t piece_dword(const Block& b, int i) {
    const int d = i >> 2;
    if (d == 12) return b.w3;
    const uint4 v = b.w[d >> 2];
    const int e = d & 3;
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// table entry of byte i of the piece, in this lane's copy: address
// byte * 256 + copy * 16 (v_perm_b32: selector values 4-7 pick bytes of the
// first source, 0-3 of the second, 0x0c gives zero)
__device__ __forceinline__ uint4 entry(const Block& b, int i, uint32_t rep) {
    const uint32_t sel = 0x0c0c0004u | (uint32_t(i & 3) << 8);
    const uint32_t a = __builtin_amdgcn_perm(rep, piece_dword(b, i), sel);
    return __builtin_bit_cast(uint4, *reinterpret_cast<lds_u32x4*>(a));
}

// codes (c, c + 1) of a group as one binary16 pair, from the entries of the
// byte holding code c (e) and of the next byte (en)
__device__ __forceinline__ uint32_t code_pair(int digit, const uint4& e, const uint4& en) {
    switch (digit) {
        case 0: return e.x;
        case 1: return __builtin_amdgcn_perm(e.y, e.x, 0x05040302u);   // e.x hi, e.y lo
        case 2: return e.y;
        case 3: return __builtin_amdgcn_perm(e.z, e.y, 0x05040302u);   // e.y hi, e.z lo
        default: return __builtin_amdgcn_perm(en.x, e.z, 0x05040100u); // e.z lo, en.x lo
    }
}

// Where a lane's A operand (activations) comes from; offsets are byte offsets
// from the start of the wave's K range (see the 2-bit-slot kernel).
template <int NT, bool XLDS>
struct XSrc;

template <int NT>
struct XSrc<NT, true> {
    uint32_t base[NT];
    uint32_t mask[NT];
    __device__ __forceinline__ uint4 get(int p, uint32_t off) const {
        return __builtin_bit_cast(uint4,
                                  *reinterpret_cast<lds_u32x4*>(base[p] + (mask[p] & off)));
    }
};

template <int NT>
struct XSrc<NT, false> {
    const uint8_t* ptr[NT];
    bool live[NT];
    __device__ __forceinline__ uint4 get(int p, uint32_t off) const {
        return live[p] ? *reinterpret_cast<const uint4*>(ptr[p] + off) : uint4{0, 0, 0, 0};
    }
};

// Decode and multiply one block into acc; off = byte offset of the block in
// the wave's K range.  For each half h: 16 windows of group 2q + h, MFMAs
// issued in batches of 4 after their operand reads.
template <int NT, bool XLDS>
__device__ __forceinline__ void compute_block(const Block& b, uint32_t rep, const XSrc<NT, XLDS>& xs,
                                              uint32_t off, float (&acc)[NT]) {
    float sc[8];
    {
        const uint32_t sw[4] = {b.s.x, b.s.y, b.s.z, b.s.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            sc[i] = __half2float(__ushort_as_half(uint16_t(sw[i >> 1] >> (16 * (i & 1)))));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float4v d[NT];
#pragma unroll
        for (int p = 0; p < NT; ++p) d[p] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w0 = 0; w0 < 16; w0 += 4) {
            uint4 av[NT][4];
#pragma unroll
            for (int p = 0; p < NT; ++p)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    // x[tok][K of group 2q + h + 8 (w0 + t) .. + 7]
                    av[p][t] = xs.get(p, off + 256u * h + 16u * (w0 + t));
            uint4 bw[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int w = w0 + t;
                uint32_t pr[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cidx = 8 * w + 2 * i;          // code index in the group
                    const int byte = 26 * h + cidx / 5;
                    const int digit = cidx % 5;
                    const uint4 e = entry(b, byte, rep);
                    const uint4 en = digit == 4 ? entry(b, byte + 1, rep) : e;
                    pr[i] = code_pair(digit, e, en);
                }
                bw[t] = uint4{pr[0], pr[1], pr[2], pr[3]};
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int p = 0; p < NT; ++p)
                    d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(half8, av[p][t]), __builtin_bit_cast(half8, bw[t]), d[p],
                        0, 0, 0);
        }
        // D row 4 * token + c holds group 2c + h of this lane's row
#pragma unroll
        for (int p = 0; p < NT; ++p)
            acc[p] += sc[h] * d[p][0] + sc[2 + h] * d[p][1] + sc[4 + h] * d[p][2] +
                      sc[6 + h] * d[p][3];
    }
}

// xstride: bytes from one 1024-block of activations to the next
template <int NR, int NT, bool XLDS>
__device__ __forceinline__ void flight(const uint8_t* wb, const uint16_t* sb, uint32_t rep,
                                       const XSrc<NT, XLDS>& xs, uint32_t off, uint32_t xstride,
                                       float (&acc)[NT]) {
    Block b[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) load_block(b[i], wb + kBlockBytes * i, sb + 8 * i);
#pragma unroll
    for (int i = 0; i < NR; ++i) compute_block<NT, XLDS>(b[i], rep, xs, off + xstride * i, acc);
}

template <int NT, bool XLDS>
__device__ __forceinline__ void flight_n(int nr, const uint8_t* wb, const uint16_t* sb,
                                         uint32_t rep, const XSrc<NT, XLDS>& xs, uint32_t off,
                                         uint32_t xstride, float (&acc)[NT]) {
    if (flight_max<NT>() >= 2 && nr >= 2)
        flight<(flight_max<NT>() >= 2 ? 2 : 1), NT, XLDS>(wb, sb, rep, xs, off, xstride, acc);
    else if (nr >= 1)
        flight<1, NT, XLDS>(wb, sb, rep, xs, off, xstride, acc);
}

// ROT (M = 1, activations in LDS): x holds the unrotated activations and
// signs their signs; the workgroup rotates them into LDS first (the 2-bit
// kernel's rotation: one wave per 1024-block, the first stage on the matrix
// cores), and workgroup 0 also writes them to x_rot.
template <int NT, bool XLDS, bool ROT>
__global__ __launch_bounds__(64 * waves<NT>()) void gemv_trit5_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, const int8_t* signs,
    uint16_t* x_rot, int m, int64_t n, int64_t k, int ksplit, int64_t rows_base, int64_t rows_rem,
    void* __restrict__ y, int y_f16) {
    static_assert(!ROT || (NT == 1 && XLDS), "the rotating prologue is for one token in LDS");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t* lut = smem;                                             // LDS address 0
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    float* red = reinterpret_cast<float*>(smem + kLutBytes);         // [wave][NT][64]
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem + kLutBytes + waves<NT>() * NT * 64 * 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int q = lane >> 4;

    // this workgroup's rows (host-side n / G and n % G), this wave's tile and blocks
    const int64_t g = blockIdx.x;
    const int64_t r0 = g * rows_base + (g < rows_rem ? g : rows_rem);
    const int64_t r1 = r0 + rows_base + (g < rows_rem ? 1 : 0);
    const int tile_slot = wave / ksplit;
    const int ks = wave - tile_slot * ksplit;
    const int tile_stride = nwaves / ksplit;
    const int tiles_here = int((r1 - r0 + 15) / 16);
    const int64_t row_bytes = (k / kBlock) * kBlockBytes;
    const int64_t groups = k / kGroup;
    const int blocks = int(k / kBlock);
    const int b0 = blocks * ks / ksplit;
    const int nb_tile = blocks * (ks + 1) / ksplit - b0;
    const int nb = tile_slot < tiles_here ? nb_tile : 0;

    // Prologue (see the 2-bit-slot kernel): activations -> LDS and the table,
    // published before any weight load is issued.
    const uint32_t xs_lds =
        uint32_t(uintptr_t((__attribute__((address_space(3))) uint16_t*)(xs)));
    const uint32_t xstride = 2048u;   // per 1024-block
    const uint32_t zero_lds = xs_lds + uint32_t(m) * uint32_t(blocks) * xstride;   // 16-byte zero pad
    if constexpr (ROT) {
        // the loads of a wave's first block go out first, the table is built
        // while they are in flight; wave w rotates blocks w, w + nwaves, ...
        rot::In rin;
        rot::load(x, signs, blocks, wave, lane, rin);
        build_lut(lut, tid, nthreads);
        if (tid == 0)
            *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(zero_lds) =
                u32x4{0, 0, 0, 0};
        rot::half8v hb[2];
        rot::h_operand(lane, hb);
        for (int blk = wave; blk < blocks; blk += nwaves) {
            if (blk != wave) rot::load(x, signs, blocks, blk, lane, rin);
            rot::run(rin, hb, lane, xs + blk * kBlock);
        }
        vm_lds_barrier();
        if (blockIdx.x == 0)
            for (int i = tid; i < blocks * 128; i += nthreads)
                reinterpret_cast<uint4*>(x_rot)[i] = reinterpret_cast<const uint4*>(xs)[i];
    } else {
        if (XLDS) {
            const int pieces = int(int64_t(m) * k / 512);   // M*K is a multiple of 1024
            for (int c = wave; c < pieces; c += nwaves)
                dma_1k(xs_lds + uint32_t(c) * 1024u, x + int64_t(c) * 512 + lane * 8);
            if (tid == 0)
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(zero_lds) =
                    u32x4{0, 0, 0, 0};
        }
        build_lut(lut, tid, nthreads);
        vm_lds_barrier();
    }

    const uint32_t rep = uint32_t(lane & 15) * 16u;   // this lane's table copy * 16
    // A-operand role: row j of A = token j / 4 of the pass, lane-group class j % 4
    const int a_tok = j >> 2;
    float acc[NT];
    XSrc<NT, XLDS> xsrc;
#pragma unroll
    for (int p = 0; p < NT; ++p) {
        acc[p] = 0.0f;
        const bool live = (j & 3) == q && (4 * p + a_tok) < m;
        const int64_t xoff = int64_t(4 * p + a_tok) * k + kBlock * b0 + 256 * q;   // halves
        if constexpr (XLDS) {
            const uint32_t lds_off = (uint32_t(4 * p + a_tok) * uint32_t(blocks) + uint32_t(b0)) *
                                         xstride + 512u * uint32_t(q);
            xsrc.base[p] = live ? xs_lds + lds_off : zero_lds;
            xsrc.mask[p] = live ? ~0u : 0u;
        } else {
            xsrc.ptr[p] = reinterpret_cast<const uint8_t*>(x + (live ? xoff : 0));
            xsrc.live[p] = live;
        }
    }

    int64_t tile = tile_slot;
    int64_t row = r0 + 16 * tile + j;
    bool row_ok = tile < tiles_here && row < r1;
    // rows past the share re-read row r0 (a valid row) and are never written
    const int64_t lrow = row_ok ? row : r0;
    const uint8_t* wb = packed + lrow * row_bytes + kBlockBytes * b0 + kPieceBytes * q;
    const uint16_t* sb = scales + lrow * groups + 8 * b0;

    constexpr int kFlight = flight_max<NT>();
    for (;;) {   // tiles of this wave (a single one unless ksplit == 1)
        for (int f = 0; f < nb; f += kFlight)
            flight_n<NT, XLDS>(nb - f, wb + kBlockBytes * f, sb + 8 * f, rep, xsrc,
                               xstride * uint32_t(f), xstride, acc);
        tile += tile_stride;
        if (ksplit > 1 || tile >= tiles_here) break;
        // whole-K tiles: write this one out and start the next
        if (row_ok) {
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                const int tok = 4 * p + q;
                if (tok < m) {
                    const int64_t oi = int64_t(tok) * n + row;
                    if (y_f16)
                        reinterpret_cast<__half*>(y)[oi] = __float2half_rn(acc[p]);
                    else
                        reinterpret_cast<float*>(y)[oi] = acc[p];
                }
            }
        }
#pragma unroll
        for (int p = 0; p < NT; ++p) acc[p] = 0.0f;
        row = r0 + 16 * tile + j;
        row_ok = row < r1;
        const int64_t nrow = row_ok ? row : r0;
        wb = packed + nrow * row_bytes + kPieceBytes * q;
        sb = scales + nrow * groups;
    }

    // D lane (j, q) holds token q of each pass for row j
#pragma unroll
    for (int p = 0; p < NT; ++p) red[(wave * NT + p) * 64 + lane] = acc[p];
    __syncthreads();
    if (ks == 0 && row_ok) {
#pragma unroll
        for (int p = 0; p < NT; ++p) {
            const int tok = 4 * p + q;
            if (tok < m) {
                float v = red[(wave * NT + p) * 64 + lane];
                for (int w2 = 1; w2 < ksplit; ++w2) v += red[((wave + w2) * NT + p) * 64 + lane];
                const int64_t oi = int64_t(tok) * n + row;
                if (y_f16)
                    reinterpret_cast<__half*>(y)[oi] = __float2half_rn(v);
                else
                    reinterpret_cast<float*>(y)[oi] = v;
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
// workgroup split K when the share is at most max_w tiles
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

// LDS bytes of a launch: table, reduction buffer, activations and a 16-byte
// zero pad
template <int NT, bool XLDS>
constexpr int64_t lds_bytes(int mt, int64_t k) {
    return kLutBytes + int64_t(waves<NT>()) * NT * 64 * 4 + (XLDS ? int64_t(mt) * k * 2 + 16 : 0);
}

template <int NT, bool XLDS, bool ROT = false>
hipError_t launch_one(const Plan& plan, const uint8_t* packed, const uint16_t* scales,
                      const uint16_t* x, const int8_t* signs, uint16_t* x_rot, int mt, int64_t n,
                      int64_t k, void* y, int y_f16, hipStream_t stream) {
    const hipError_t e =
        allow_lds(reinterpret_cast<const void*>(gemv_trit5_kernel<NT, XLDS, ROT>), int(kLdsLimit));
    if (e != hipSuccess) return e;
    size_t lds = size_t(lds_bytes<NT, XLDS>(mt, k));
    // ask for more than half of the CU's LDS so that two workgroups never share a CU
    if (lds < size_t(kLdsLimit / 2 + 1024)) lds = size_t(kLdsLimit / 2 + 1024);
    hipLaunchKernelGGL((gemv_trit5_kernel<NT, XLDS, ROT>), dim3(unsigned(plan.grid)),
                       dim3(64 * plan.waves), lds, stream, packed, scales, x, signs, x_rot, mt, n,
                       k, plan.ksplit, n / plan.grid, n % plan.grid, y, y_f16);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_nt(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int mt,
                     int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    const Plan plan = make_plan(n, waves<NT>());
    // activations go to LDS (with a 16-byte zero pad) when they fit beside the
    // table and the reduction buffer
    const int64_t budget = kLdsLimit - kLutBytes - int64_t(waves<NT>()) * NT * 64 * 4;
    if (int64_t(mt) * k * 2 + 16 <= budget)
        return launch_one<NT, true>(plan, packed, scales, x, nullptr, nullptr, mt, n, k, y, y_f16,
                                    stream);
    return launch_one<NT, false>(plan, packed, scales, x, nullptr, nullptr, mt, n, k, y, y_f16,
                                 stream);
}

}  // namespace

// tl_linear at M = 1 in one launch: the rotated activations must fit in LDS
// beside the table
bool linear_m1_trit5_fits(int64_t m, int64_t n, int64_t k) {
    (void)n;
    return m == 1 && lds_bytes<1, true>(1, k) <= kLdsLimit;
}

hipError_t launch_linear_m1_trit5(const uint8_t* packed, const uint16_t* scales,
                                  const uint16_t* x, const int8_t* signs, uint16_t* x_rot,
                                  int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    const Plan plan = make_plan(n, waves<1>());
    return launch_one<1, true, true>(plan, packed, scales, x, signs, x_rot, 1, n, k, y, y_f16,
                                     stream);
}

hipError_t launch_gemv_trit5(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream) {
    const int64_t y_elem = y_f16 ? 2 : 4;
    // up to 16 tokens per launch, 4 per pass
    for (int64_t m0 = 0; m0 < m; m0 += 16) {
        const int mt = int(m - m0 < 16 ? m - m0 : 16);
        const uint16_t* xs = x + m0 * k;
        void* ys = static_cast<uint8_t*>(y) + m0 * n * y_elem;
        hipError_t e;
        if (mt <= 4)
            e = launch_nt<1>(packed, scales, xs, mt, n, k, ys, y_f16, stream);
        else if (mt <= 8)
            e = launch_nt<2>(packed, scales, xs, mt, n, k, ys, y_f16, stream);
        else
            e = launch_nt<4>(packed, scales, xs, mt, n, k, ys, y_f16, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace tl
