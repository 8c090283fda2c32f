// Decode chains at M = 1, 2-bit-slot packing: one persistent launch runs a
// list of linears (tl_linear_chain), each the rotation of its input followed
// by the ternary product, as tl_linear does (page "A 27-billion model that
// fits in 8.6 GB", paragraphs 2 and 3: the rotation folded into the weights is
// applied to the activations of every linear at run time).
//
// Why.  At M = 1 a linear is a pure weight stream, and one launch per linear
// pays, every time, the ramp-up and drain of the stream, the launch gap and a
// prologue (input load, rotation, activation images) during which little of
// the weight stream is in flight.  The weights never depend on the
// activations, so here every workgroup requests the first steps of the next
// linear's weights as soon as it has finished its share of the current one,
// before it waits for that linear's input: the weight stream continues
// through the boundary.
//
// Work.  The grid is one workgroup per CU; every workgroup runs the linears
// in order and owns the same contiguous slice of rows of each (rows split as
// evenly as possible), computed exactly as the single-linear kernel of
// gemv_m1.hip does (the same decode, matrix-core diagonal products and fixed
// summation order, so each linear's result is bit-identical to tl_linear's).
//
// Dependencies.  A linear whose input lies in the output of an earlier linear
// of the chain (the plan records which) waits until every workgroup has written
// its rows of that output: after its stores a workgroup makes them visible at
// device scope (release fence) and adds 1 to the producer's counter in the
// caller's sync buffer; the consumer's first thread polls the counter until it
// reaches the grid size, then acquires.  The poll is bounded: after the plan's
// limit, or as soon as another workgroup has reported an error, it records
// the error (2 + the waiting linear's index, first error kept) in the sync
// buffer and every workgroup leaves the chain.  Linears whose inputs are ready
// at launch do not wait.  The last workgroup to leave resets every counter to
// zero, so the sync buffer is ready for the next call; the error word stays
// until the caller clears it.  The waits need every workgroup resident at once
// (one per CU, forced by the LDS size): a GPU shared with other work can make
// them time out, which is reported, never a hang.
//
// Wave 0's first thread does the polling; wave 0 issues its own early weight
// requests after the poll, so that its polling loads do not queue behind them.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "../../include/tl.h"
#include "m1_decode.h"
#include "rotate_lds.h"
#include "tl_internal.h"

namespace tl {
namespace {

using namespace m1;

constexpr uint32_t kChainMagic = 0x4E484354u;
constexpr int kChainFL = 6;       // weight steps per flight
constexpr int kChainCross = 4;    // steps of the next linear loaded during the current one
constexpr int kChainMaxFlights = 3;   // flights of one linear (unrolled: no loop-carried loads)
constexpr uint32_t kDefaultPolls = 1u << 20;
constexpr int kFlagOffset = int(kLdsLimit) - 16;   // LDS word: this workgroup leaves the chain
// per-segment partial sums of the current linear (at most kMaxSegsPerChunk
// segments) at a fixed place, below the flag and above everything the next
// linear's rotation and images use, so that wave 0 can add them up while the
// other waves go on
constexpr int kRedOffset = kFlagOffset - kMaxSegsPerChunk * 16;

struct ChainHead {
    uint32_t magic;
    int32_t count;
    int32_t grid;           // workgroups the plan was encoded for (CUs of the device)
    uint32_t max_polls;     // polls of a dependency wait before it gives up
    uint32_t pad[12];
};
struct ChainOp {
    const uint8_t* packed;
    const uint16_t* scales;
    const uint16_t* x;
    const int8_t* signs;
    uint16_t* x_rot;        // may be null
    void* y;
    int32_t n, k;
    int32_t dep;            // index of the linear whose output is x, or -1
    int32_t y_f16;
};
static_assert(sizeof(ChainHead) == 64 && sizeof(ChainOp) == 64, "plan layout");

// A linear as one workgroup sees it: its rows, its slot's segment range
// (block-major, one chunk) and the buffer resources of its weight rows.
struct OpState {
    int nb, rows, beg, end, steps, flights, row_bytes, groups;
    __amdgpu_buffer_rsrc_t wsrc, ssrc;
};

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache policy of the accesses that cross workgroups (a linear's output,
// read as a later linear's input): coherent at device scope (sc1), so no
// cache has to be written back or invalidated for them.
constexpr int kDeviceScope = 16;
// Cache policy of the weight and scale loads: read once per chain, streamed
// (nontemporal) so that they do not push the linears' inputs out of the caches.
constexpr int kNonTemporal = 2;

// s_waitcnt immediate: vector memory count 0, the other counters not waited
constexpr int kVmcntZero = 0x0F70;

template <int FL, int CROSS, int MAXF>
__global__ __launch_bounds__(kThreads) void chain_kernel(const uint8_t* __restrict__ plan, int count,
                                                         uint32_t* sync) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int* leave = reinterpret_cast<int*>(smem + kFlagOffset);
    const ChainHead* head = reinterpret_cast<const ChainHead*>(plan);
    const ChainOp* ops = reinterpret_cast<const ChainOp*>(plan + sizeof(ChainHead));
    uint32_t* done = sync;                 // [count]: workgroups finished with each linear
    uint32_t* exited = sync + count;       // workgroups that left the chain
    uint32_t* err = sync + count + 1;      // 0, or the first error

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int slot_in_wave = col >> 2;
    const int ip = lane & 3;
    const int u = 4 * ip + q;
    const int slot = 4 * wave + slot_in_wave;
    const bool diag = q == slot_in_wave;
    const int bid = int(blockIdx.x);
    const int grid = int(gridDim.x);

    auto state = [&](const ChainOp& op) {
        OpState st;
        st.nb = op.k / kBlock;
        const int base = op.n / grid, rem = op.n % grid;
        const int64_t r0 = int64_t(bid) * base + min(bid, rem);
        st.rows = base + (bid < rem ? 1 : 0);
        st.row_bytes = op.k / 4;
        st.groups = op.k / kGroup;
        const int segs = st.rows * st.nb;
        st.beg = slot * segs / kSlots;
        st.end = (slot + 1) * segs / kSlots;
        st.steps = (segs + kSlots - 1) / kSlots;   // of the slot with the most
        st.flights = (st.steps + FL - 1) / FL;
        st.wsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(op.packed + r0 * st.row_bytes),
                                                    0, st.rows * st.row_bytes, kRsrcWord3);
        st.ssrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(op.scales + r0 * st.groups),
                                                    0, st.rows * st.groups * 2, kRsrcWord3);
        return st;
    };

    // The weight ring: wv[t], sv[t] hold step t of the flight being computed.
    // As soon as step t is consumed, the same registers receive step t of the
    // next flight, or, during a linear's last flight, step t < CROSS of the
    // next linear's first flight (its steps CROSS.. are loaded after that
    // linear's rotation, which needs their registers): FL steps per slot stay
    // in flight within a linear, CROSS across its boundary.
    uint4 wv[FL];
    uint32_t sv[FL];
    // where the loads of a flight go: first segment, its block and row, and
    // the linear's resources (selected among two linears with uniform selects)
    struct Loads {
        int f0, b, r, rc, end, row_bytes, groups;
        __amdgpu_buffer_rsrc_t wsrc, ssrc;
        bool live;
    };
    auto loads_of = [&](const OpState& s, int f, bool live) {
        Loads l;
        l.rc = s.rows > 0 ? s.rows : 1;
        l.f0 = s.beg + f * FL;
        l.b = l.f0 / l.rc;
        l.r = l.f0 - l.b * l.rc;
        l.end = s.end;
        l.row_bytes = s.row_bytes;
        l.groups = s.groups;
        l.wsrc = s.wsrc;
        l.ssrc = s.ssrc;
        l.live = live;
        return l;
    };
    // load step t of l into wv[t], sv[t] (steps past the slot's range, or of a
    // dead flight, read nothing: out-of-range offsets return zeros); t is a
    // constant after unrolling
    auto load_step = [&](Loads& l, int t, bool want = true) {
        const bool ok = want && l.live && l.f0 + t < l.end;
        const uint32_t wo = ok ? uint32_t(l.r * l.row_bytes + 256 * l.b + 16 * u) : kOob;
        const uint32_t so = ok ? uint32_t((l.r * l.groups + 8 * l.b + 2 * ip) * 2) : kOob;
        wv[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(l.wsrc, wo, 0, kNonTemporal));
        sv[t] = __builtin_amdgcn_raw_buffer_load_b32(l.ssrc, so, 0, kNonTemporal);
        // keep the loads in step order: the compiler then waits for exactly
        // the step it consumes (else it hoists the refills above the steps
        // and waits for every load in flight)
        __builtin_amdgcn_sched_barrier(0);
        if (++l.r == l.rc) {
            l.r = 0;
            ++l.b;
        }
    };
    auto load_steps = [&](Loads l, int t_lo, int t_hi) {
#pragma unroll
        for (int t = 0; t < FL; ++t)
            if (t >= t_lo && t < t_hi)
                load_step(l, t);
            else if (++l.r == l.rc) {
                l.r = 0;
                ++l.b;
            }
    };
    // step t of flight f of the current linear, then the refill of its
    // registers; a[], rf, rx, ry: the activation images of block cur_b
    auto step = [&](const OpState& st, int& b, int& r, int f0, Loads& nl, const uint8_t* img,
                    const uint8_t* rec, float* red, int t, bool live, bool refill, int& cur_b,
                    half8 (&a)[8], float& rf, float& rx, float& ry) {
        const int rc = st.rows > 0 ? st.rows : 1;
        const bool ok = f0 + t < st.end;
        // steps past every slot's range (workgroup-uniform) only refill the ring
        if (live) {
        if (ok && b != cur_b) {   // slot-uniform; rare (slots run block-major)
            const uint8_t* src = img + b * kImgBlock + u * kImgLane;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                a[j] = __builtin_bit_cast(half8,
                                          *reinterpret_cast<const lds_u32x4*>(lds_addr(src + 16 * j)));
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
        const float part =
            (h2f(sv[t] & 0xFFFFu) * (pick(dx, ip) + rx) + h2f(sv[t] >> 16) * (pick(dy, ip) + ry)) * rf;
        if (diag && ok) red[(r * st.nb + b) * 4 + ip] = part;
        if (++r == rc) {
            r = 0;
            ++b;
        }
        }
        load_step(nl, t, refill);
    };

    const bool plan_ok = head->magic == kChainMagic && head->count == count && head->grid == grid;
    if (!plan_ok) {
        if (tid == 0) {
            uint32_t zero = 0;
            __hip_atomic_compare_exchange_strong(err, &zero, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        const uint32_t max_polls = head->max_polls;
        OpState st = state(ops[0]);
        load_steps(loads_of(st, 0, true), 0, CROSS);
        for (int i = 0; i < count; ++i) {
            const ChainOp op = ops[i];
            const int nb = st.nb;
            uint16_t* xrot = reinterpret_cast<uint16_t*>(smem);
            uint8_t* img = smem + nb * 2048;
            uint8_t* rec = img + nb * kImgBlock;
            float* red = reinterpret_cast<float*>(smem + kRedOffset);
            // the next linear: its first CROSS steps are loaded during this
            // linear's last flight, except by wave 0, which stores this
            // linear's output and publishes it (a wait for its stores would
            // also wait for such loads) and may poll for the next input: wave 0
            // loads them once that is done
            const bool has_next = i + 1 < count;
            const OpState nx = has_next ? state(ops[i + 1]) : st;

            // the input: when an earlier linear of the chain writes it, wait
            // until every workgroup has written its rows
            if (op.dep >= 0) {
                if (wave == 0) {
                    if (lane == 0) {
                        int bad = 0;
                        uint32_t polls = 0;
                        while (ld_agent(done + op.dep) < uint32_t(grid)) {
                            if (ld_agent(err) != 0u || polls++ >= max_polls) {
                                bad = 1;
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                        }
                        if (bad) {
                            uint32_t zero = 0;
                            __hip_atomic_compare_exchange_strong(err, &zero, uint32_t(2 + i),
                                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT);
                        }
                        *leave = bad;
                    }
                }
                lds_barrier();
                if (__builtin_amdgcn_readfirstlane(*leave)) break;
            }
            if (i > 0 && wave == 0) load_steps(loads_of(st, 0, true), 0, CROSS);

            // rotation of the input into LDS as tl_linear's kernel does it (x_rot
            // written by workgroup 0; the input read at device scope), then the
            // activation images
            {
                // one block's input in registers at a time: this kernel holds
                // the next linear's first weight steps through the rotation
                rot::half8v hb[2];
                rot::h_operand(lane, hb);
                for (int blk = wave; blk < nb; blk += kWaves) {
                    rot::In rin;
                    rot::load<kDeviceScope>(op.x, op.signs, nb, blk, lane, rin);
                    rot::run(rin, hb, lane, xrot + blk * kBlock);
                }
                uint4 xraw[4];
                lds_barrier();
                if (bid == 0 && op.x_rot)
                    for (int j = tid; j < nb * 128; j += kThreads)
                        reinterpret_cast<uint4*>(op.x_rot)[j] = reinterpret_cast<const uint4*>(xrot)[j];
                load_x_lds(xrot, nb, tid, xraw);
                if (wave * 64 < nb * 32) build_pass(xraw, nb, tid, img, rec);
                lds_barrier();
            }

            // the weight stream: the first flight's steps not loaded during the
            // previous linear (their registers stay free during the rotation)
            // (nothing else may be in flight before them: a real wait
            // instruction, which the compiler's wait placement accounts for)
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            load_steps(loads_of(st, 0, true), CROSS, FL);
            int cur_b = -1;
            half8 a[8];
            float rf = 0.0f, rx = 0.0f, ry = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) a[j] = half8{};
            // (the flights are unrolled: a loop would carry loads in flight
            // across its back edge, and the compiler then waits for all of
            // them at the top of every flight)
#pragma unroll
            for (int f = 0; f < MAXF; ++f) {
                if (f < st.flights) {
                    const int f0 = st.beg + f * FL;
                    const int rc = st.rows > 0 ? st.rows : 1;
                    int b = f0 / rc, r = f0 - (f0 / rc) * rc;
                    const bool last = f + 1 == st.flights;
                    const int left = st.steps - f * FL;
                    Loads nl = last ? loads_of(nx, 0, has_next && wave != 0) : loads_of(st, f + 1, true);
#pragma unroll
                    for (int t = 0; t < FL; ++t)
                        step(st, b, r, f0, nl, img, rec, red, t, t < left, !last || t < CROSS, cur_b,
                             a, rf, rx, ry);
                }
            }
            if (st.flights == 0 && has_next && wave != 0) load_steps(loads_of(nx, 0, true), 0, CROSS);
            lds_barrier();

            // this workgroup's rows of y, added by wave 0 in a fixed order
            // (blocks ascending, the four columns of each block), stored with
            // device-scope stores, then published: once they are complete,
            // the linear's counter goes up
            if (wave == 0) {
                const int64_t r0 = int64_t(bid) * (op.n / grid) + min(bid, op.n % grid);
                const int esz = op.y_f16 ? 2 : 4;
                const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint8_t*>(op.y) + r0 * esz, 0, st.rows * esz, kRsrcWord3);
                for (int r = lane; r < st.rows; r += 64) {
                    const float4* pr = reinterpret_cast<const float4*>(red + r * nb * 4);
                    float v = 0.0f;
                    for (int b = 0; b < nb; ++b) {
                        const float4 p = pr[b];
                        v = (((v + p.x) + p.y) + p.z) + p.w;
                    }
                    if (op.y_f16)
                        __builtin_amdgcn_raw_buffer_store_b16(uint16_t(f2h(v)), ys, uint32_t(2 * r),
                                                              0, kDeviceScope);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ys,
                                                              uint32_t(4 * r), 0, kDeviceScope);
                }
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
                if (lane == 0)
                    __hip_atomic_fetch_add(done + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            st = nx;
        }
    }

    // leave: loads of a linear the chain did not reach may still be in
    // flight; then the last workgroup out resets the counters for the next
    // call
    // (this also completes the counter updates before the exit count)
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    if (tid == 0) {
        const uint32_t before =
            __hip_atomic_fetch_add(exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == uint32_t(grid - 1)) {
            for (int j = 0; j < count; ++j)
                __hip_atomic_store(done + j, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(exited, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// LDS below the partial sums: rotated input, then the images and records
int64_t lds_need(int64_t nb) { return nb * 2048 + nb * kImgBlock + nb * 4 * kRecBytes; }

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    if (!a || !b) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + uintptr_t(b_bytes) && b0 < a0 + uintptr_t(a_bytes);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int64_t chain_plan_bytes(int64_t count) { return int64_t(sizeof(ChainHead)) + count * int64_t(sizeof(ChainOp)); }

int64_t chain_sync_bytes(int64_t count) { return ((4 * (count + 2) + 15) / 16) * 16; }

int chain_encode(const tl_chain_op* ops, int32_t count, void* plan_out) {
    const int grid = cu_count();
    struct Buf {
        const void* p;
        int64_t bytes;
    };
    // per linear: inputs (codes, scales, x, signs) and outputs (y, x_rot)
    auto inputs = [&](const tl_chain_op& o, Buf (&b)[4]) {
        b[0] = {o.packed, o.N * (o.K / 4)};
        b[1] = {o.scales, o.N * (o.K / kGroup) * 2};
        b[2] = {o.x, o.K * 2};
        b[3] = {o.signs, o.K};
    };
    auto outputs = [&](const tl_chain_op& o, Buf (&b)[2]) {
        b[0] = {o.y, o.N * (o.y_dtype == TL_F16 ? 2 : 4)};
        b[1] = {o.x_rot, o.K * 2};
    };
    for (int i = 0; i < count; ++i) {
        const tl_chain_op& o = ops[i];
        if (!o.packed || !o.scales || !o.x || !o.signs || !o.y) return TL_ERR_NULL;
        if (o.fmt != TL_FMT_SLOT2) return TL_ERR_FORMAT;
        if (o.y_dtype != TL_F32 && o.y_dtype != TL_F16) return TL_ERR_DTYPE;
        if (o.N < 1 || o.N > (int64_t(1) << 24) || o.K < kBlock || o.K % kBlock != 0 ||
            o.K / kBlock * 32 > kThreads)
            return TL_ERR_SHAPE;
        const int64_t nb = o.K / kBlock, rows = (o.N + grid - 1) / grid;
        if (rows * nb > int64_t(kSlots) * kChainFL * kChainMaxFlights || lds_need(nb) > kRedOffset ||
            rows * (o.K / 4) >= (int64_t(1) << 31))
            return TL_ERR_SHAPE;
        if (!aligned16(o.packed) || !aligned16(o.scales) || !aligned16(o.x) || !aligned16(o.signs) ||
            !aligned16(o.y) || !aligned16(o.x_rot))
            return TL_ERR_ALIGN;
    }
    // An output may overlap nothing else of the chain, except that it may be,
    // exactly, the input x of later linears (which then wait for it).
    ChainHead* head = static_cast<ChainHead*>(plan_out);
    ChainOp* dst = reinterpret_cast<ChainOp*>(static_cast<uint8_t*>(plan_out) + sizeof(ChainHead));
    for (int i = 0; i < count; ++i) {
        const tl_chain_op& o = ops[i];
        Buf out[2];
        outputs(o, out);
        if (overlap(out[0].p, out[0].bytes, out[1].p, out[1].bytes)) return TL_ERR_ALIAS;
        for (int j = 0; j < count; ++j) {
            const tl_chain_op& p = ops[j];
            Buf in[4], po[2];
            inputs(p, in);
            outputs(p, po);
            for (const Buf& w : out) {
                for (int e = 0; e < 4; ++e) {
                    if (!overlap(w.p, w.bytes, in[e].p, in[e].bytes)) continue;
                    // x of a later linear inside this binary16 y: it waits for it
                    const uintptr_t x0 = reinterpret_cast<uintptr_t>(p.x),
                                    y0 = reinterpret_cast<uintptr_t>(o.y);
                    const bool feeds = e == 2 && j > i && w.p == o.y && o.y_dtype == TL_F16 &&
                                       x0 >= y0 && x0 + uintptr_t(p.K * 2) <= y0 + uintptr_t(o.N * 2);
                    if (!feeds) return TL_ERR_ALIAS;
                }
                if (j != i)
                    for (const Buf& v : po)
                        if (overlap(w.p, w.bytes, v.p, v.bytes)) return TL_ERR_ALIAS;
            }
        }
    }
    for (int i = 0; i < count; ++i) {
        const tl_chain_op& o = ops[i];
        int dep = -1;   // the earlier linear whose y holds x (outputs never overlap: one at most)
        for (int j = 0; j < i; ++j)
            if (ops[j].y_dtype == TL_F16 && overlap(ops[j].y, ops[j].N * 2, o.x, o.K * 2)) dep = j;
        dst[i] = ChainOp{o.packed, o.scales, o.x, o.signs, o.x_rot, o.y, int32_t(o.N), int32_t(o.K),
                         dep, o.y_dtype == TL_F16 ? 1 : 0};
    }
    *head = ChainHead{};
    head->magic = kChainMagic;
    head->count = count;
    head->grid = grid;
    head->max_polls = kDefaultPolls;
    return TL_OK;
}

hipError_t launch_chain(const void* plan, int32_t count, uint32_t* sync, hipStream_t stream) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(chain_kernel<kChainFL, kChainCross, kChainMaxFlights>),
                                   int(kLdsLimit));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chain_kernel<kChainFL, kChainCross, kChainMaxFlights>), dim3(unsigned(cu_count())), dim3(kThreads),
                       kLdsLimit, stream, static_cast<const uint8_t*>(plan), int(count), sync);
    return hipGetLastError();
}

}  // namespace tl
