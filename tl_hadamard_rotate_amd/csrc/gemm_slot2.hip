// Prefill ternary g128 GEMM for the 2-bit-slot packing:
//   y[m, n] = sum_k x[m, k] * code[n, k] * S[n, k/128].
// The weights reach the matrix cores without an fp16 copy in LDS: their packed
// bytes are staged in LDS (0.25 byte per weight), and every wave reads the
// bytes of its own 64 weight rows and decodes them in registers, straight into
// the B operand of v_mfma_f32_32x32x16_f16, as exact binary16 values code * S
// (a code in {-1, 0, 1} times a binary16 scale is a binary16 number).  The
// activations, which every wave of a row of the tile shares, are staged in LDS
// as they are.  Prompt processing is the bottleneck the pages name for slower
// chips (page "A 27-billion model that fits in 8.6 GB", paragraph 4).
//
// Tiling: a workgroup of 8 waves (two per SIMD) computes a 256 x 256 output
// tile (M x N); wave w owns the 128 x 64 sub-tile (w / 4, w % 4): 4 x 2 MFMA
// tiles of 32 x 32, 128 fp32 accumulators per lane.  Per K step (64) a wave
// issues 32 MFMAs, decodes 64 weights per lane and reads 16 KB of activations
// from LDS: 16 KB of LDS traffic per MFLOP, against 50 KB for 64 x 64
// sub-tiles with the weights staged in LDS as well.
//
// K order inside an MFMA is free as long as the A and B operands agree, and
// it is chosen so that a lane's weights of a step are 8 contiguous packed
// bytes under one scale: K runs in blocks of 256 (4 steps); in block T, lane
// half q = lane / 32 covers K [256T + 128q, +128), one scale group; in step t
// of the block, K slice s (0..3) of element e is
// K = 256T + 128q + 32t + 8s + e.  The activation tile of step t is staged to
// match: row r holds, as 16-byte chunk 4q + s, x[r][256T + 128q + 32t + 8s ..].
// Chunks are stored with c -> c ^ ((r >> 1) & 7), so that the 16 lanes a
// 128-bit LDS read serves per cycle (16 rows, one chunk) hit 16 distinct bank
// groups.
//
// Decode: a byte of the packing holds 4 digits (d = code + 1).  One v_perm
// spreads byte b of a packed word to [b, b, b >> 2, b >> 2]; masking with
// 0x03 per byte and setting bit 2 of bytes 1 and 3 gives the selector
// [d0, d0 + 4, d1, d1 + 4]; a second v_perm with that selector picks, per
// byte, from the 8 bytes [lo(S), 0, lo(S), 0, hi(S) ^ 0x80, 0, hi(S), 0], which
// yields the binary16 pair (code0 * S, code1 * S) exactly (digit 3, which the
// packer never writes, decodes to 0).  About 1.6 VALU operations per weight.
//
// Activations, packed weights and scales go from memory straight into LDS
// (global_load_lds) through four stages, three steps ahead of their use, with
// one barrier per step; the scales of a block of 4 steps one block ahead.
// Workgroups are mapped so that each XCD (blockIdx % 8) runs a contiguous run
// of tiles, N fastest: concurrent workgroups of an XCD share activation rows
// in that XCD's L2.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "tl_internal.h"

namespace tl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr int BM = 256, BN = 256, BK = 64;
// 8 waves: two per SIMD, 128 x 64 sub-tiles, 128 accumulators (the other wave
// of a SIMD issues while one waits; 8-18 % faster than 4 waves of 128 x 128
// sub-tiles with the whole register file, measured over the MLP shapes)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesN = kWaves / 2;          // waves along N (two along M)
constexpr int NJ = 16 / kWaves;              // 32-wide MFMA column tiles per wave
constexpr int kRegs = 4 * NJ * 16;           // accumulators per lane
constexpr int kALoads = 32 / kWaves;         // 1 KB activation loads per wave per step
constexpr int kBLoads = 16 / kWaves;         // 256 B weight loads per wave per step
constexpr int kVmWait = kALoads + kBLoads;   // fewest loads a wave issues in a step
constexpr int kAStage = BM * BK * 2;   // 32 KB
constexpr int kStages = 4;
constexpr int kTileFloats = BM * BN;   // partial sums of one tile
constexpr int kBStage = BN * 16;     // 4 KB: packed weights of one step
constexpr int kSStage = BN * 4;      // 1 KB: scales of one block
constexpr int kLds = kStages * (kAStage + kBStage) + 2 * kSStage;   // 146 KB
static_assert(kLds <= 160 * 1024, "LDS");

// byte offset of 16-byte chunk c of row r in a [rows][64 halves] tile
__device__ __forceinline__ uint32_t swz(int r, int c) {
    return uint32_t(r) * 128u + 16u * uint32_t(c ^ ((r >> 1) & 7));
}

// the two v_perm source words for one binary16 scale S:
// hi word bytes [hi(S) ^ 0x80, 0, hi(S), 0], lo word bytes [lo(S), 0, lo(S), 0]
struct ScaleSel {
    uint32_t hi, lo;
};

__device__ __forceinline__ ScaleSel scale_sel(uint32_t s) {
    const uint32_t lo = s & 0xFFu, hi = (s >> 8) & 0xFFu;
    return ScaleSel{(hi ^ 0x80u) | (hi << 16), lo | (lo << 16)};
}

// codes 8h .. 8h + 7 of a packed dword (code i in bits 2i..2i+1) -> 4
// binary16 pairs: out[i] = (code 8h + 2i, code 8h + 2i + 1) * S.  mask holds
// 0x03030303, bits 0x04000400, both in VGPRs, so that (y & mask) | bits is
// one v_and_or_b32 (VOP3 takes no literal here and at most one SGPR).
__device__ __forceinline__ void decode8(uint32_t w, int h, ScaleSel sc, uint32_t mask, uint32_t bits,
                                        uint32_t* out) {
    const uint32_t w2 = w >> 2;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const uint32_t y = __builtin_amdgcn_perm(w2, w, 0x04040000u + 0x01010101u * uint32_t(2 * h + b));
        out[2 * b] = __builtin_amdgcn_perm(sc.hi, sc.lo, (y & mask) | bits);
        out[2 * b + 1] = __builtin_amdgcn_perm(sc.hi, sc.lo, ((y >> 4) & mask) | bits);
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4))) void gemm_slot2_kernel(
    const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t m, int64_t n,
    int64_t k, void* __restrict__ y, int y_f16, int tiles_n, int tiles, int t0, int chunk_a,
    int splits, int chunk_b, float* __restrict__ ws, const float* __restrict__ row_scale) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t st0 = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(smem)));

    // Work items.  Tiles [0, t0) are computed whole by blocks [0, 8 chunk_a);
    // each tile of [t0, tiles) is split along K into `splits` parts, item v of
    // blocks [8 chunk_a, ...) being part v % splits of tile t0 + v / splits.
    // XCD-aware order in both ranges: XCD (blockIdx % 8) takes a contiguous
    // run of items, N fastest, so that concurrent workgroups of an XCD share
    // activation rows (and the parts of a tile sit on one XCD).
    int tile, sp = 0, slot = 0;
    bool split = false;
    if (int(blockIdx.x) < 8 * chunk_a) {
        tile = int(blockIdx.x & 7) * chunk_a + int(blockIdx.x >> 3);
        if (tile >= t0) return;
    } else {
        const int u = int(blockIdx.x) - 8 * chunk_a;
        slot = (u & 7) * chunk_b + (u >> 3);
        if (slot >= (tiles - t0) * splits) return;
        tile = t0 + slot / splits;
        sp = slot % splits;
        split = splits > 1;
    }
    const int64_t m0 = int64_t(tile / tiles_n) * BM;
    const int64_t n0 = int64_t(tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nblk = int(k / 256);
    const int ksteps = 4 * nblk;
    // K range of this item, in units of 8 steps (the loop's unroll)
    const int units = nblk / 2;
    const int u0 = split ? sp * units / splits : 0, u1 = split ? (sp + 1) * units / splits : units;
    const int tb = 8 * u0;   // first step
    const uint32_t groups = uint32_t(k / kGroup);
    const uint32_t row_bytes = uint32_t(k / 4);

    const int wm = (wave / kWavesN) * 128, wn = (wave % kWavesN) * (32 * NJ);
    const int q = lane >> 5;

    // LDS: four activation and four weight stages (one step each), two scale
    // stages (one block each)
    const uint32_t a_lds = st0, b_lds = st0 + kStages * kAStage, s_lds = b_lds + kStages * kBStage;

    // Everything the loop reads from memory goes straight to LDS
    // (global_load_lds: lane i of a wave's load lands at LDS base + size * i),
    // so the loop holds no register loads and the only waits on memory are
    // the explicit ones before each barrier.
    //
    // Activations, 1 KB per load: wave w stages tile rows 32 w .. 32 w + 31,
    // eight rows per load (four loads); load u puts row 32 w + 8 u + i / 8,
    // physical chunk i % 8, which holds logical chunk (i % 8) ^ ((row >> 1) &
    // 7), i.e. ((i % 8) ^ (i / 16 + 4 (u % 2))).
    uint32_t aoff[kALoads];   // byte offsets
#pragma unroll
    for (int u = 0; u < kALoads; ++u) {
        const int64_t r = m0 + (256 / kWaves) * wave + 8 * u + (lane >> 3);
        const uint32_t gm = uint32_t(r < m ? r : m - 1);   // rows past M copy row M-1
        const uint32_t c = uint32_t((lane & 7) ^ ((lane >> 4) + 4 * (u & 1)));
        aoff[u] = 2u * (gm * uint32_t(k) + 128u * (c >> 2) + 8u * (c & 3u));
    }
    const char* xb = reinterpret_cast<const char*>(x);
    auto dma_a = [&](uint32_t stage, int t, int u) {   // load u of step t
        const uint32_t o = 512u * uint32_t(t >> 2) + 64u * uint32_t(t & 3);
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(uintptr_t)(xb + (aoff[u] + o)),
            (__attribute__((address_space(3))) void*)(uintptr_t)(stage + (32768u / kWaves) * uint32_t(wave) + 1024u * u),
            16, 0, 0);
    };
    // Packed weights, 4 bytes per lane and load: the weight stage of step t
    // (step t % 4 of block T = t / 4) holds, per tile row n and K half h, the
    // 8 bytes (32 codes) at byte 64 T + 32 h + 8 (t % 4) of the row:
    // [n][h][8 B].  Wave w loads rows 32 w .. 32 w + 31, 16 rows per 256-byte
    // load (two loads): lane i of load v takes row 32 w + 16 v + i / 4, half
    // (i / 2) % 2, dword i % 2.
    uint32_t boff[kBLoads];
#pragma unroll
    for (int v = 0; v < kBLoads; ++v) {
        const int64_t r = n0 + (256 / kWaves) * wave + 16 * v + (lane >> 2);
        const uint32_t gn = uint32_t(r < n ? r : n - 1);   // rows past N decode row N-1
        boff[v] = gn * row_bytes + 32u * uint32_t((lane >> 1) & 1) + 4u * uint32_t(lane & 1);
    }
    auto dma_b = [&](uint32_t stage, int t, int v) {   // load v of step t
        const uint32_t o = 64u * uint32_t(t >> 2) + 8u * uint32_t(t & 3);
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(uintptr_t)(packed + (boff[v] + o)),
            (__attribute__((address_space(3))) void*)(uintptr_t)(stage + (4096u / kWaves) * uint32_t(wave) + 256u * v),
            4, 0, 0);
    };
    // Scales, per block: the scale stage holds the dword of groups
    // (2T, 2T + 1) of each tile row, [n][4 B]; waves 0..3 load rows 64 w .. +63.
    uint32_t soff;
    {
        const int64_t r = n0 + 64 * (wave & 3) + lane;
        const uint32_t gn = uint32_t(r < n ? r : n - 1);
        soff = 2u * gn * groups;
    }
    const char* sb = reinterpret_cast<const char*>(scales);
    auto dma_s = [&](uint32_t stage, int t_blk) {   // waves 0..3, 64 rows each
        if (wave >= 4) return;
        __builtin_amdgcn_global_load_lds(
            (__attribute__((address_space(1))) void*)(uintptr_t)(sb + (soff + 4u * uint32_t(t_blk))),
            (__attribute__((address_space(3))) void*)(uintptr_t)(stage + 256u * uint32_t(wave)), 4, 0, 0);
    };

    uint32_t mask = 0x03030303u, bits = 0x04000400u;
    asm volatile("" : "+v"(mask), "+v"(bits));   // keep both in VGPRs

    // this lane's weight rows: column l % 32 of MFMA tiles j = 0..3
    const uint32_t brow = uint32_t(wn + (lane & 31));

    // Pipeline.  During step t the MFMAs read step t's activation stage; the
    // fragments and weights of the next K slice are read from LDS (and the
    // weights decoded) while a slice's MFMAs run, step t + 1's first slice
    // during step t's last.  Step t loads, spread over its K slices, step
    // t + 3's activations and weights into the stages step t - 1 used and, in
    // a block's first step, the next block's scales.  At the end of step t,
    // s_waitcnt vmcnt(6) leaves at most the wave's 6 newest loads outstanding;
    // every step issues at least 6, so every load of step t - 1 is complete,
    // and after the barrier all that step t + 1 reads is in LDS: activations
    // and weights of step t + 2 and scales of the block of t + 2.  Stage
    // reuse: the stages step t + 3 takes were last read in step t - 1 (its
    // activations) and step t - 2 (its weights); the scale stage of block
    // T + 1 (two stages) in step 4T - 1.  The loop is unrolled over 8 steps,
    // a whole period of every stage rotation, so that all LDS addresses are
    // compile-time offsets and the compiler can see that no LDS read aliases
    // a load in flight (else it would wait for the loads).  K is a multiple of
    // 1024, so the number of steps is a multiple of 16 and the loop below
    // needs no tail; loads past the end re-read the last step or block.
    uint32_t stg_a[kStages];   // activation stage of step t + i
    uint32_t stg_b[kStages];   // weight stage of step t + i
    uint32_t stg_s[2];         // scale stage of block t / 4 + i
#pragma unroll
    for (int i = 0; i < kStages; ++i) stg_a[i] = a_lds + uint32_t(i) * kAStage;
#pragma unroll
    for (int i = 0; i < kStages; ++i) stg_b[i] = b_lds + uint32_t(i) * kBStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) stg_s[i] = s_lds + uint32_t(i) * kSStage;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int u = 0; u < kALoads; ++u) dma_a(stg_a[i], tb + i, u);
#pragma unroll
        for (int v = 0; v < kBLoads; ++v) dma_b(stg_b[i], tb + i, v);
    }
    dma_s(stg_s[0], tb >> 2);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);

    auto read_af = [&](half8 (&af)[4], uint32_t base, int s) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = __builtin_bit_cast(
                half8, *reinterpret_cast<lds_u32x4*>(base + swz(wm + 32 * i + (lane & 31), 4 * q + s)));
    };
    // this lane's 8 bytes of a step for rows j
    auto read_b = [&](uint2 (&w)[NJ], uint32_t stage) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            w[j] = __builtin_bit_cast(uint2, *reinterpret_cast<lds_u32x2*>(stage + (brow + 32u * j) * 16u + 8u * q));
    };
    auto read_sc = [&](ScaleSel (&sc)[NJ], uint32_t stage) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            sc[j] = scale_sel(*reinterpret_cast<__attribute__((address_space(3))) uint16_t*>(
                stage + (brow + 32u * j) * 4u + 2u * q));
    };
    // The same reads inside the loop, written out: as plain C++ the compiler
    // cannot tell them from reads of a stage a load is filling and makes
    // them wait for every load in flight.  Each block waits for its own
    // reads (and the LDS reads before them) before it ends.
    auto read_b_asm = [&](uint2 (&w)[NJ], uint32_t stage) {
        const uint32_t a = stage + brow * 16u + 8u * q;
        uint64_t r[4];
        if (NJ == 4)
            asm volatile(
                "ds_read_b64 %0, %4\n\t"
                "ds_read_b64 %1, %4 offset:512\n\t"
                "ds_read_b64 %2, %4 offset:1024\n\t"
                "ds_read_b64 %3, %4 offset:1536\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                : "v"(a)
                : "memory");
        else
            asm volatile(
                "ds_read_b64 %0, %2\n\t"
                "ds_read_b64 %1, %2 offset:512\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r[0]), "=&v"(r[1])
                : "v"(a)
                : "memory");
#pragma unroll
        for (int j = 0; j < NJ; ++j) w[j] = __builtin_bit_cast(uint2, r[j]);
    };
    auto read_sc_asm = [&](ScaleSel (&sc)[NJ], uint32_t stage) {
        const uint32_t a = stage + brow * 4u + 2u * q;
        uint32_t r[4];
        if (NJ == 4)
            asm volatile(
                "ds_read_u16 %0, %4\n\t"
                "ds_read_u16 %1, %4 offset:128\n\t"
                "ds_read_u16 %2, %4 offset:256\n\t"
                "ds_read_u16 %3, %4 offset:384\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                : "v"(a)
                : "memory");
        else
            asm volatile(
                "ds_read_u16 %0, %2\n\t"
                "ds_read_u16 %1, %2 offset:128\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(r[0]), "=&v"(r[1])
                : "v"(a)
                : "memory");
#pragma unroll
        for (int j = 0; j < NJ; ++j) sc[j] = scale_sel(r[j]);
    };
    // B operands of slice s (codes 8s .. 8s + 7 of the step's 32 per row)
    auto decode_bf = [&](half8 (&bf)[NJ], const uint2 (&w)[NJ], const ScaleSel (&sc)[NJ], int s) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint32_t o[4];
            decode8(s < 2 ? w[j].x : w[j].y, s & 1, sc[j], mask, bits, o);
            bf[j] = __builtin_bit_cast(half8, u32x4{o[0], o[1], o[2], o[3]});
        }
    };

    // operands of slice s sit in buffer s % 2; weights of step t in rb[t % 2]
    half8 af[2][4], bf[2][NJ];
    uint2 rb[2][NJ];
    ScaleSel sc[2][NJ];   // blocks T and T + 1
    read_sc(sc[0], stg_s[0]);
    read_b(rb[0], stg_b[0]);
    read_af(af[0], stg_a[0], 0);
    decode_bf(bf[0], rb[0], sc[0], 0);

    float16v acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // one K step t (step TT of block T, scale selectors of T in sc[TB])
    auto step = [&](int t, auto tt_c, auto tb_c) {
        constexpr int TT = decltype(tt_c)::value, TB = decltype(tb_c)::value;
        constexpr int SL = TT & 1;   // weight registers of step t
        const int t3 = t + 3 < ksteps ? t + 3 : ksteps - 1;
        const int b1 = (t >> 2) + 1 < nblk ? (t >> 2) + 1 : nblk - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int nb = (s + 1) & 1;
            // loads, pinned at the slice start: the compiler makes a load into
            // LDS wait for every LDS read in flight, here only the previous
            // slice's, which this slice's MFMAs need anyway
#pragma unroll
            for (int u = s * kALoads / 4; u < (s + 1) * kALoads / 4; ++u) dma_a(stg_a[3], t3, u);
            if (kBLoads == 4 || !(s & 1)) dma_b(stg_b[3], t3, kBLoads == 4 ? s : s >> 1);
            if (s == 2 && TT == 0) dma_s(stg_s[1], b1);
            __builtin_amdgcn_sched_barrier(0);
            if (s < 3) {
                read_af(af[nb], stg_a[0], s + 1);
                decode_bf(bf[nb], rb[SL], sc[TB], s + 1);
            } else {
                // slice 0 of step t + 1 (its stages are complete since the
                // barrier that ended step t - 1)
                read_b_asm(rb[SL ^ 1], stg_b[1]);
                if (TT == 3) read_sc_asm(sc[TB ^ 1], stg_s[1]);
                read_af(af[nb], stg_a[1], 0);
                decode_bf(bf[nb], rb[SL ^ 1], sc[TT == 3 ? TB ^ 1 : TB], 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][i], bf[s & 1][j], acc[i][j],
                                                                       0, 0, 0);
        }
        {   // rotate the stages
            const uint32_t a0 = stg_a[0];
#pragma unroll
            for (int i = 0; i + 1 < kStages; ++i) stg_a[i] = stg_a[i + 1];
            stg_a[kStages - 1] = a0;
            const uint32_t b0 = stg_b[0];
#pragma unroll
            for (int i = 0; i + 1 < kStages; ++i) stg_b[i] = stg_b[i + 1];
            stg_b[kStages - 1] = b0;
            if (TT == 3) {
                const uint32_t s0 = stg_s[0];
                stg_s[0] = stg_s[1];
                stg_s[1] = s0;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        static_assert(kVmWait == 6, "the wait below counts the loads of a step");
        asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" : : : "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;
    auto block = [&](int t_blk, auto tb_c) {
        const int t = 4 * t_blk;
        step(t, C0{}, tb_c);
        step(t + 1, C1{}, tb_c);
        step(t + 2, C2{}, tb_c);
        step(t + 3, C3{}, tb_c);
    };
    for (int t_blk = 2 * u0; t_blk < 2 * u1; t_blk += 2) {
        block(t_blk, C0{});
        block(t_blk + 1, C1{});
    }

    // loads into stages nobody reads may still be in flight: drain them before
    // the workgroup can end and its LDS be handed to another
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");

    if (split) {
        // part of a K-split tile: its partial sums go to this item's
        // workspace slot, [register][thread]; gemm_slot2_reduce adds the parts
        float* mine = ws + size_t(slot) * kTileFloats;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[((i * NJ + j) * 16 + r) * kThreads + tid] = acc[i][j][r];
        return;
    }

    // lane holds D[8 * (r / 4) + 4 * (lane / 32) + r % 4][lane % 32] of each
    // 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
                const int64_t col = n0 + wn + 32 * j + (lane & 31);
                if (row < m && col < n) {
                    const float v = row_scale ? acc[i][j][r] * row_scale[row] : acc[i][j][r];
                    if (y_f16)
                        reinterpret_cast<__half*>(y)[row * n + col] = __float2half_rn(v);
                    else
                        reinterpret_cast<float*>(y)[row * n + col] = v;
                }
            }
}

// Sum of the K parts of the split tiles, in part order (so the result does
// not depend on the order the parts ran in), stored to y.  Block b handles
// accumulator register e = b % kRegs of split tile t0 + b / kRegs for all
// kThreads threads of the GEMM's workgroup layout: thread tid holds that
// register of wave tid / 64 at the same place as there.
__global__ __launch_bounds__(kThreads) void gemm_slot2_reduce(const float* __restrict__ ws,
                                                              int64_t m, int64_t n, void* __restrict__ y,
                                                              int y_f16, int tiles_n, int t0, int splits,
                                                              const float* __restrict__ row_scale) {
    const int tt = int(blockIdx.x) / kRegs, e = int(blockIdx.x) % kRegs;
    const int tile = t0 + tt;
    const int64_t m0 = int64_t(tile / tiles_n) * BM;
    const int64_t n0 = int64_t(tile % tiles_n) * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = (wave / kWavesN) * 128, wn = (wave % kWavesN) * (32 * NJ), q = lane >> 5;
    const float* parts = ws + size_t(tt) * splits * kTileFloats + e * kThreads + tid;
    float sum = parts[0];
    for (int p = 1; p < splits; ++p) sum += parts[size_t(p) * kTileFloats];
    const int i = e / (16 * NJ), j = (e / 16) % NJ, r = e % 16;
    const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * q + (r & 3);
    const int64_t col = n0 + wn + 32 * j + (lane & 31);
    if (row < m && col < n) {
        if (row_scale) sum *= row_scale[row];
        if (y_f16)
            reinterpret_cast<__half*>(y)[row * n + col] = __float2half_rn(sum);
        else
            reinterpret_cast<float*>(y)[row * n + col] = sum;
    }
}

}  // namespace

bool gemm_slot2_fits(int64_t m, int64_t n, int64_t k) {
    // K a multiple of 1024 (see the loop); 32-bit byte offsets
    return m >= 1 && n >= 1 && k >= 1024 && k % 1024 == 0 && m * k < (int64_t(1) << 31) &&
           n * (k / 4) < (int64_t(1) << 32);
}

namespace {

// K split of the tiles that do not fill a whole round of workgroups (one per
// CU).  Cost model in units of the loop (8 steps, about 14 us of one
// workgroup): rounds of parts of ceil(units / splits) units, plus the partial
// sums written and read back (256 KB per part, about 0.01 unit at the HBM
// rate) and the reducing launch (0.3 unit).  At most kMaxSplitItems parts in
// all, so the partial sums never need more than 64 MiB of workspace.
constexpr int64_t kMaxSplitItems = 256;

Gemm2Plan plan_split(int64_t tiles, int units, int cus) {
    const int64_t rem = tiles % cus;
    Gemm2Plan best{tiles, tiles, 1};
    if (rem == 0) return best;
    double best_cost = units;
    for (int s = 2; s <= 16 && s <= units && rem * s <= kMaxSplitItems; ++s) {
        const int64_t rounds = (rem * s + cus - 1) / cus;
        const double cost = double(rounds) * double((units + s - 1) / s) + 0.01 * double(rem * s) + 0.3;
        if (cost < best_cost - 0.5) {
            best_cost = cost;
            best = Gemm2Plan{tiles, tiles - rem, s};
        }
    }
    return best;
}

}  // namespace

Gemm2Plan gemm_slot2_plan(int64_t m, int64_t n, int64_t k) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    return plan_split(tiles, int(k / 512), cu_count());
}

int64_t gemm_slot2_workspace_bytes(int64_t m, int64_t n, int64_t k) {
    const Gemm2Plan pl = gemm_slot2_plan(m, n, k);
    return pl.splits > 1 ? (pl.tiles - pl.t0) * pl.splits * int64_t(kTileFloats) * 4 : 0;
}

hipError_t launch_gemm_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16, void* ws,
                             int64_t ws_bytes, hipStream_t stream, const float* row_scale) {
    if (!gemm_slot2_fits(m, n, k)) return hipErrorInvalidValue;
    const Gemm2Plan pl = gemm_slot2_plan(m, n, k);
    const int64_t items = (pl.tiles - pl.t0) * pl.splits;
    if (pl.splits > 1 && (ws == nullptr || ws_bytes < items * int64_t(kTileFloats) * 4))
        return hipErrorInvalidValue;
    hipError_t e = allow_lds(reinterpret_cast<const void*>(gemm_slot2_kernel), kLds);
    if (e != hipSuccess) return e;
    const int64_t tiles_n = (n + BN - 1) / BN;
    float* part = pl.splits > 1 ? static_cast<float*>(ws) : nullptr;
    const int64_t chunk_a = (pl.t0 + 7) / 8, chunk_b = (items + 7) / 8;
    hipLaunchKernelGGL(gemm_slot2_kernel, dim3(unsigned(8 * (chunk_a + chunk_b))), dim3(kThreads),
                       size_t(kLds), stream, packed, scales, x, m, n, k, y, y_f16, int(tiles_n),
                       int(pl.tiles), int(pl.t0), int(chunk_a), pl.splits, int(chunk_b), part, row_scale);
    if (pl.splits > 1) {
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(gemm_slot2_reduce, dim3(unsigned(kRegs * (pl.tiles - pl.t0))),
                           dim3(kThreads), 0, stream, part, m, n, y, y_f16, int(tiles_n),
                           int(pl.t0), pl.splits, row_scale);
    }
    return hipGetLastError();
}

}  // namespace tl
