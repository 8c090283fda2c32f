// Prefill products for every packing, and the layout of their workspace.
// The matrix-core kernels read 2-bit slots; the dense trit and 1-bit packings
// are rewritten as 2-bit slots once per call (one pass over the weights, small
// next to the product: prompt processing is compute-bound, so the denser
// format only has to be read once) into the start of the caller's workspace.
// The fp16 product's K-split partial sums follow at the next 256-byte
// boundary.
#include "tl_internal.h"

namespace tl {
namespace {

int64_t rewrite_bytes(int64_t n, int64_t k, int fmt) {
    return fmt == 1 ? 0 : ((n * (k / 4) + 255) / 256) * 256;
}

// the 2-bit-slot weights the kernels read: the packed codes themselves, or
// their rewrite into the workspace
hipError_t slot2_weights(const uint8_t* packed, int fmt, int64_t n, int64_t k, void* ws,
                         const uint8_t** out, hipStream_t stream) {
    if (fmt == 1) {
        *out = packed;
        return hipSuccess;
    }
    uint8_t* s2 = static_cast<uint8_t*>(ws);
    const hipError_t e = fmt == 0 ? launch_trit5_to_slot2(packed, n, k, s2, stream)
                                  : launch_bit1_to_slot2(packed, n, k, s2, stream);
    *out = s2;
    return e;
}

}  // namespace

bool gemm_fits(int64_t m, int64_t n, int64_t k) { return gemm_slot2_fits(m, n, k); }

int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int fmt, bool bf16) {
    return rewrite_bytes(n, k, fmt) + (bf16 ? 0 : gemm_slot2_workspace_bytes(m, n, k));
}

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, void* ws,
                       int64_t ws_bytes, hipStream_t stream) {
    if (!gemm_fits(m, n, k) || ws_bytes < gemm_workspace_bytes(m, n, k, fmt, false))
        return hipErrorInvalidValue;
    const uint8_t* s2 = nullptr;
    const hipError_t e = slot2_weights(packed, fmt, n, k, ws, &s2, stream);
    if (e != hipSuccess) return e;
    const int64_t off = rewrite_bytes(n, k, fmt);
    void* part = ws ? static_cast<uint8_t*>(ws) + off : nullptr;
    return launch_gemm_slot2(s2, scales, x, m, n, k, y, y_f16, part, ws_bytes - off, stream);
}

hipError_t launch_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int fmt,
                            const uint16_t* x, int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            void* ws, int64_t ws_bytes, hipStream_t stream) {
    if (!gemm_fits(m, n, k) || ws_bytes < gemm_workspace_bytes(m, n, k, fmt, true))
        return hipErrorInvalidValue;
    const uint8_t* s2 = nullptr;
    const hipError_t e = slot2_weights(packed, fmt, n, k, ws, &s2, stream);
    if (e != hipSuccess) return e;
    return launch_gemm_bf16_slot2(s2, scales, x, m, n, k, y, y_f16, stream);
}

}  // namespace tl
