// C ABI of libtl: argument validation, then one launch on the caller's stream.
// Every check runs on the host before anything is enqueued, so a rejected call
// leaves every output untouched.
#include <stdint.h>

#include <cstdlib>
#include <initializer_list>
#include <mutex>
#include <string>
#include <utility>

#include "tl_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxRows = int64_t(1) << 24;     // M and N
constexpr int64_t kMaxElems = int64_t(1) << 36;    // M*K, N*K and M*N
constexpr int32_t kMaxChain = 65536;               // linears in one chain

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + uintptr_t(b_bytes) && b0 < a0 + uintptr_t(a_bytes);
}

bool known_fmt(int32_t fmt) {
    return fmt == TL_FMT_TRIT5 || fmt == TL_FMT_SLOT2 || fmt == TL_FMT_BIT1;
}

int64_t row_bytes(int64_t k, int32_t fmt) {
    return fmt == TL_FMT_TRIT5 ? (k / TL_GROUP) * 26 : fmt == TL_FMT_BIT1 ? k / 8 : k / 4;
}

tl_status launched(hipError_t e) {
    if (e == hipSuccess) return TL_OK;
    g_last_error = hipGetErrorString(e);
    return TL_ERR_LAUNCH;
}

bool pack_shape_ok(int64_t n, int64_t k) {
    return n >= 1 && n <= kMaxRows && k >= TL_GROUP && k % TL_GROUP == 0 && k <= TL_MAX_K &&
           n * k <= kMaxElems;
}

bool layer_shape_ok(int64_t m, int64_t n, int64_t k) {
    return m >= 1 && m <= kMaxRows && n >= 1 && n <= kMaxRows && k >= TL_BLOCK &&
           k % TL_BLOCK == 0 && k <= TL_MAX_K && m * k <= kMaxElems && n * k <= kMaxElems &&
           m * n <= kMaxElems;
}

tl_status check_layer(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                      const uint16_t* x_rot, int64_t m, int64_t n, int64_t k, void* y,
                      int32_t y_dtype) {
    if (!packed || !scales || !x_rot || !y) return TL_ERR_NULL;
    if (!layer_shape_ok(m, n, k)) return TL_ERR_SHAPE;
    if (!known_fmt(fmt)) return TL_ERR_FORMAT;
    if (y_dtype != TL_F32 && y_dtype != TL_F16) return TL_ERR_DTYPE;
    if (!aligned16(packed) || !aligned16(scales) || !aligned16(x_rot) || !aligned16(y))
        return TL_ERR_ALIGN;
    const int64_t y_bytes = m * n * (y_dtype == TL_F32 ? 4 : 2);
    if (overlap(y, y_bytes, packed, n * row_bytes(k, fmt)) ||
        overlap(y, y_bytes, scales, n * (k / TL_GROUP) * 2) || overlap(y, y_bytes, x_rot, m * k * 2))
        return TL_ERR_ALIAS;
    return TL_OK;
}

// workspace of a prefill product: present when needed, large enough, aligned,
// and overlapping none of the call's buffers
tl_status check_workspace(int64_t need, const void* ws, int64_t ws_bytes,
                          std::initializer_list<std::pair<const void*, int64_t>> bufs) {
    if (need == 0) return TL_OK;
    if (!ws || ws_bytes < need) return TL_ERR_WORKSPACE;
    if (!aligned16(ws)) return TL_ERR_ALIGN;
    for (const auto& b : bufs)
        if (b.first && overlap(ws, need, b.first, b.second)) return TL_ERR_ALIAS;
    return TL_OK;
}

// TL_DEBUG=1: count the packed bytes that are not valid encodings before a
// call that decodes them; a device int per GPU holds the count
bool debug_on() {
    const char* e = std::getenv("TL_DEBUG");
    return e && e[0] == '1' && e[1] == '\0';
}

tl_status debug_check(const uint8_t* packed, int64_t n, int64_t k, int32_t fmt, hipStream_t stream) {
    if (!debug_on() || fmt == TL_FMT_BIT1) return TL_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return launched(e);
    if (cs != hipStreamCaptureStatusNone) return TL_OK;   // no waiting inside a capture
    static std::mutex mu;
    static int32_t* counters[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return launched(e);
    if (dev < 0 || dev >= 64) return launched(hipErrorInvalidDevice);
    if (!counters[dev]) {
        void* p = nullptr;
        e = hipMalloc(&p, 256);
        if (e != hipSuccess) return launched(e);
        counters[dev] = static_cast<int32_t*>(p);
    }
    int32_t bad = 0;
    e = hipMemsetAsync(counters[dev], 0, sizeof(int32_t), stream);
    if (e == hipSuccess) e = tl::launch_count_invalid(packed, n, k, fmt, counters[dev], stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(&bad, counters[dev], sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return launched(e);
    if (bad != 0) {
        g_last_error = std::to_string(bad) + " packed bytes are not valid encodings";
        return TL_ERR_DATA;
    }
    return TL_OK;
}

}  // namespace

extern "C" {

int64_t tl_packed_bytes(int64_t N, int64_t K, int32_t fmt) {
    if (N < 1 || K < TL_GROUP || K % TL_GROUP != 0) return -1;
    if (!known_fmt(fmt)) return -1;
    return N * row_bytes(K, fmt);
}

tl_status tl_pack(const int8_t* codes, int64_t N, int64_t K, int32_t fmt, uint8_t* packed,
                  int32_t* bad_count, hipStream_t stream) {
    if (!codes || !packed) return TL_ERR_NULL;
    if (!pack_shape_ok(N, K)) return TL_ERR_SHAPE;
    if (!known_fmt(fmt)) return TL_ERR_FORMAT;
    if (!aligned16(codes) || !aligned16(packed)) return TL_ERR_ALIGN;
    if (bad_count && (reinterpret_cast<uintptr_t>(bad_count) & 3u)) return TL_ERR_ALIGN;
    const int64_t pb = N * row_bytes(K, fmt);
    if (overlap(packed, pb, codes, N * K)) return TL_ERR_ALIAS;
    if (bad_count && (overlap(bad_count, 4, codes, N * K) || overlap(bad_count, 4, packed, pb)))
        return TL_ERR_ALIAS;
    return launched(tl::launch_pack(codes, N, K, fmt, packed, bad_count, stream));
}

tl_status tl_unpack(const uint8_t* packed, int64_t N, int64_t K, int32_t fmt, int8_t* codes,
                    hipStream_t stream) {
    if (!codes || !packed) return TL_ERR_NULL;
    if (!pack_shape_ok(N, K)) return TL_ERR_SHAPE;
    if (!known_fmt(fmt)) return TL_ERR_FORMAT;
    if (!aligned16(codes) || !aligned16(packed)) return TL_ERR_ALIGN;
    if (overlap(packed, N * row_bytes(K, fmt), codes, N * K)) return TL_ERR_ALIAS;
    const tl_status st = debug_check(packed, N, K, fmt, stream);
    if (st != TL_OK) return st;
    return launched(tl::launch_unpack(packed, N, K, fmt, codes, stream));
}

tl_status tl_hadamard_rotate(const uint16_t* x, const int8_t* signs, int64_t M, int64_t K,
                             uint16_t* x_rot, hipStream_t stream) {
    if (!x || !signs || !x_rot) return TL_ERR_NULL;
    if (!(M >= 1 && M <= kMaxRows && K >= TL_BLOCK && K % TL_BLOCK == 0 && K <= TL_MAX_K &&
          M * K <= kMaxElems))
        return TL_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(signs) || !aligned16(x_rot)) return TL_ERR_ALIGN;
    const int64_t bytes = M * K * 2;
    if (x_rot != x && overlap(x_rot, bytes, x, bytes)) return TL_ERR_ALIAS;
    if (overlap(x_rot, bytes, signs, K)) return TL_ERR_ALIAS;
    return launched(tl::launch_hadamard(x, signs, M, K, x_rot, stream));
}

tl_status tl_gemv(const uint8_t* packed, const uint16_t* scales, int32_t fmt, const uint16_t* x_rot,
                  int64_t M, int64_t N, int64_t K, void* y, int32_t y_dtype, hipStream_t stream) {
    tl_status st = check_layer(packed, scales, fmt, x_rot, M, N, K, y, y_dtype);
    if (st != TL_OK) return st;
    st = debug_check(packed, N, K, fmt, stream);
    if (st != TL_OK) return st;
    return launched(
        tl::launch_gemv(packed, scales, fmt, x_rot, M, N, K, y, y_dtype == TL_F16, stream));
}

int64_t tl_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t fmt) {
    if (!layer_shape_ok(M, N, K) || !known_fmt(fmt) || !tl::gemm_fits(M, N, K)) return -1;
    return tl::gemm_workspace_bytes(M, N, K, fmt, false);
}

int64_t tl_gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t fmt) {
    if (!layer_shape_ok(M, N, K) || !known_fmt(fmt) || !tl::gemm_fits(M, N, K)) return -1;
    return tl::gemm_workspace_bytes(M, N, K, fmt, true);
}

tl_status tl_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t* out) {
    if (!out) return TL_ERR_NULL;
    if (!layer_shape_ok(M, N, K) || !tl::gemm_fits(M, N, K)) return TL_ERR_SHAPE;
    const tl::Gemm2Plan p = tl::gemm_slot2_plan(M, N, K);
    out[0] = p.tiles;
    out[1] = p.t0;
    out[2] = p.splits;
    return TL_OK;
}

tl_status tl_gemm(const uint8_t* packed, const uint16_t* scales, int32_t fmt, const uint16_t* x_rot,
                  int64_t M, int64_t N, int64_t K, void* y, int32_t y_dtype, void* workspace,
                  int64_t workspace_bytes, hipStream_t stream) {
    tl_status st = check_layer(packed, scales, fmt, x_rot, M, N, K, y, y_dtype);
    if (st != TL_OK) return st;
    if (!tl::gemm_fits(M, N, K)) return TL_ERR_SHAPE;
    const int64_t need = tl::gemm_workspace_bytes(M, N, K, fmt, false);
    st = check_workspace(need, workspace, workspace_bytes,
                         {{packed, N * row_bytes(K, fmt)}, {scales, N * (K / TL_GROUP) * 2},
                          {x_rot, M * K * 2}, {y, M * N * (y_dtype == TL_F32 ? 4 : 2)}});
    if (st != TL_OK) return st;
    st = debug_check(packed, N, K, fmt, stream);
    if (st != TL_OK) return st;
    return launched(tl::launch_gemm(packed, scales, fmt, x_rot, M, N, K, y, y_dtype == TL_F16,
                                    workspace, workspace_bytes, stream));
}

tl_status tl_gemm_noalloc(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                          const uint16_t* x_rot, int64_t M, int64_t N, int64_t K, void* y,
                          int32_t y_dtype, hipStream_t stream) {
    const tl_status st = check_layer(packed, scales, fmt, x_rot, M, N, K, y, y_dtype);
    if (st != TL_OK) return st;
    if (!tl::gemm_fits(M, N, K)) return TL_ERR_SHAPE;
    const int64_t need = tl::gemm_workspace_bytes(M, N, K, fmt, false);
    if (need > int64_t(TL_GEMM_NOALLOC_MAX_WORKSPACE)) return TL_ERR_WORKSPACE;
    void* ws = nullptr;
    int64_t ws_bytes = 0;
    const hipError_t e = tl::noalloc_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return launched(e);
    return launched(tl::launch_gemm(packed, scales, fmt, x_rot, M, N, K, y, y_dtype == TL_F16, ws,
                                    ws_bytes, stream));
}

tl_status tl_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                       const uint16_t* x_rot, int64_t M, int64_t N, int64_t K, void* y,
                       int32_t y_dtype, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream) {
    tl_status st = check_layer(packed, scales, fmt, x_rot, M, N, K, y, y_dtype);
    if (st != TL_OK) return st;
    if (!tl::gemm_fits(M, N, K)) return TL_ERR_SHAPE;
    const int64_t need = tl::gemm_workspace_bytes(M, N, K, fmt, true);
    st = check_workspace(need, workspace, workspace_bytes,
                         {{packed, N * row_bytes(K, fmt)}, {scales, N * (K / TL_GROUP) * 2},
                          {x_rot, M * K * 2}, {y, M * N * (y_dtype == TL_F32 ? 4 : 2)}});
    if (st != TL_OK) return st;
    st = debug_check(packed, N, K, fmt, stream);
    if (st != TL_OK) return st;
    return launched(tl::launch_gemm_bf16(packed, scales, fmt, x_rot, M, N, K, y,
                                         y_dtype == TL_F16, workspace, workspace_bytes, stream));
}

tl_status tl_linear(const uint8_t* packed, const uint16_t* scales, int32_t fmt, const uint16_t* x,
                    const int8_t* signs, int64_t M, int64_t N, int64_t K, uint16_t* x_rot, void* y,
                    int32_t y_dtype, void* workspace, int64_t workspace_bytes,
                    hipStream_t stream) {
    tl_status st = check_layer(packed, scales, fmt, x, M, N, K, y, y_dtype);
    if (st != TL_OK) return st;
    if (!signs || !x_rot) return TL_ERR_NULL;
    if (!aligned16(signs) || !aligned16(x_rot)) return TL_ERR_ALIGN;
    const int64_t xb = M * K * 2, yb = M * N * (y_dtype == TL_F32 ? 4 : 2);
    if (overlap(x_rot, xb, x, xb) || overlap(x_rot, xb, signs, K) ||
        overlap(x_rot, xb, packed, N * row_bytes(K, fmt)) ||
        overlap(x_rot, xb, scales, N * (K / TL_GROUP) * 2) || overlap(x_rot, xb, y, yb) ||
        overlap(y, yb, signs, K))
        return TL_ERR_ALIAS;
    const bool prefill = M >= 64;
    if (prefill) {
        if (!tl::gemm_fits(M, N, K)) return TL_ERR_SHAPE;
        st = check_workspace(tl::gemm_workspace_bytes(M, N, K, fmt, false), workspace,
                             workspace_bytes,
                             {{packed, N * row_bytes(K, fmt)}, {scales, N * (K / TL_GROUP) * 2},
                              {x, xb}, {signs, K}, {x_rot, xb}, {y, yb}});
        if (st != TL_OK) return st;
    }
    st = debug_check(packed, N, K, fmt, stream);
    if (st != TL_OK) return st;
    const int y_f16 = y_dtype == TL_F16;
    if (fmt == TL_FMT_SLOT2 && tl::linear_m1_slot2_fits(M, N, K))
        return launched(
            tl::launch_linear_m1_slot2(packed, scales, x, signs, x_rot, N, K, y, y_f16, stream));
    if (fmt == TL_FMT_BIT1 && tl::linear_m1_bit1_fits(M, N, K))
        return launched(
            tl::launch_linear_m1_bit1(packed, scales, x, signs, x_rot, N, K, y, y_f16, stream));
    if (fmt == TL_FMT_TRIT5 && tl::linear_m1_trit5_fits(M, N, K))
        return launched(
            tl::launch_linear_m1_trit5(packed, scales, x, signs, x_rot, N, K, y, y_f16, stream));
    hipError_t e = tl::launch_hadamard(x, signs, M, K, x_rot, stream);
    if (e != hipSuccess) return launched(e);
    e = prefill ? tl::launch_gemm(packed, scales, fmt, x_rot, M, N, K, y, y_f16, workspace,
                                  workspace_bytes, stream)
                : tl::launch_gemv(packed, scales, fmt, x_rot, M, N, K, y, y_f16, stream);
    return launched(e);
}

int64_t tl_chain_plan_bytes(int32_t count) {
    return count >= 1 && count <= kMaxChain ? tl::chain_plan_bytes(count) : -1;
}

int64_t tl_chain_sync_bytes(int32_t count) {
    return count >= 1 && count <= kMaxChain ? tl::chain_sync_bytes(count) : -1;
}

tl_status tl_chain_encode(const tl_chain_op* ops, int32_t count, void* plan, int64_t plan_bytes) {
    if (!ops || !plan) return TL_ERR_NULL;
    if (count < 1 || count > kMaxChain || plan_bytes < tl::chain_plan_bytes(count))
        return TL_ERR_SHAPE;
    return static_cast<tl_status>(tl::chain_encode(ops, count, plan));
}

tl_status tl_linear_chain(const void* plan, int32_t count, uint32_t* sync, hipStream_t stream) {
    if (!plan || !sync) return TL_ERR_NULL;
    if (count < 1 || count > kMaxChain) return TL_ERR_SHAPE;
    if (!aligned16(plan) || !aligned16(sync)) return TL_ERR_ALIGN;
    if (overlap(plan, tl::chain_plan_bytes(count), sync, tl::chain_sync_bytes(count)))
        return TL_ERR_ALIAS;
    return launched(tl::launch_chain(plan, count, sync, stream));
}

tl_status tl_quantize(const float* w, const int8_t* signs, int64_t N, int64_t K, int8_t* codes,
                      uint16_t* scales, hipStream_t stream) {
    if (!w || !signs || !codes || !scales) return TL_ERR_NULL;
    if (!(N >= 1 && N <= kMaxRows && K >= TL_BLOCK && K % TL_BLOCK == 0 && K <= TL_MAX_K &&
          N * K <= kMaxElems))
        return TL_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(signs) || !aligned16(codes) || !aligned16(scales))
        return TL_ERR_ALIGN;
    const int64_t wb = N * K * 4, cb = N * K, sb = N * (K / TL_GROUP) * 2;
    if (overlap(codes, cb, w, wb) || overlap(codes, cb, signs, K) || overlap(codes, cb, scales, sb) ||
        overlap(scales, sb, w, wb) || overlap(scales, sb, signs, K))
        return TL_ERR_ALIAS;
    return launched(tl::launch_quantize(w, signs, N, K, codes, scales, stream));
}

const char* tl_status_str(tl_status status) {
    switch (status) {
        case TL_OK: return "TL_OK";
        case TL_ERR_NULL: return "TL_ERR_NULL";
        case TL_ERR_SHAPE: return "TL_ERR_SHAPE";
        case TL_ERR_FORMAT: return "TL_ERR_FORMAT";
        case TL_ERR_ALIGN: return "TL_ERR_ALIGN";
        case TL_ERR_ALIAS: return "TL_ERR_ALIAS";
        case TL_ERR_LAUNCH: return "TL_ERR_LAUNCH";
        case TL_ERR_DTYPE: return "TL_ERR_DTYPE";
        case TL_ERR_WORKSPACE: return "TL_ERR_WORKSPACE";
        case TL_ERR_DATA: return "TL_ERR_DATA";
    }
    return "TL_ERR_UNKNOWN";
}

const char* tl_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
