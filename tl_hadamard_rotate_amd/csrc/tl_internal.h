// Internal declarations shared by the HIP translation units of libtl.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tl.h"

namespace tl {

constexpr int kBlock = 1024;        // Hadamard block width
constexpr int kGroup = 128;         // weights per binary16 scale
constexpr int kTrit5GroupBytes = 26;

// Compute units of the current device (looked up once per device).
int cu_count();
// Let `kernel` use `bytes` of dynamic LDS on the current device (once per
// kernel and device; thread-safe).
hipError_t allow_lds(const void* kernel, int bytes);

hipError_t launch_pack(const int8_t* codes, int64_t n, int64_t k, int fmt,
                       uint8_t* packed, int32_t* bad_count, hipStream_t stream);
hipError_t launch_unpack(const uint8_t* packed, int64_t n, int64_t k, int fmt,
                         int8_t* codes, hipStream_t stream);
hipError_t launch_hadamard(const uint16_t* x, const int8_t* signs, int64_t m, int64_t k,
                           uint16_t* out, hipStream_t stream);
hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int fmt,
                       const uint16_t* x, int64_t m, int64_t n, int64_t k,
                       void* y, int y_f16, hipStream_t stream);
hipError_t launch_gemv_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream);
// M = 1 decode GEMV of the 2-bit-slot packing (matrix-core diagonal form);
// usable when gemv_m1_slot2_fits(m, n, k)
bool gemv_m1_slot2_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream);
// The same kernel with the activation rotation fused in front (x unrotated;
// x_rot receives the rotated activations); usable when linear_m1_slot2_fits
bool linear_m1_slot2_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_m1_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                  const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k,
                                  void* y, int y_f16, hipStream_t stream);
// The same two for the 1-bit packing (each 16 bits spread into the 2-bit-slot
// word of the same weights)
bool gemv_m1_bit1_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_m1_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                               int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream);
bool linear_m1_bit1_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_m1_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                 const int8_t* signs, uint16_t* x_rot, int64_t n, int64_t k,
                                 void* y, int y_f16, hipStream_t stream);
// 2 <= M <= 16 decode GEMV of the 2-bit-slot packing (tokens on the
// matrix-core rows, up to 8 per workgroup, two token groups in one launch);
// usable when gemv_mt_slot2_fits(m, n, k)
bool gemv_mt_slot2_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_mt_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                                int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                                hipStream_t stream);
// the same kernel for the 1-bit packing (each 16 bits of codes spread into a
// 2-bit-slot word); usable when gemv_mt_bit1_fits(m, n, k)
bool gemv_mt_bit1_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_mt_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                               int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                               hipStream_t stream);
// Dense trits at M = 1 with the rotation fused in front (x unrotated; x_rot
// receives the rotated activations); usable when linear_m1_trit5_fits
bool linear_m1_trit5_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_m1_trit5(const uint8_t* packed, const uint16_t* scales,
                                  const uint16_t* x, const int8_t* signs, uint16_t* x_rot,
                                  int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream);
hipError_t launch_gemv_trit5(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream);
// The dense trit packing rewritten as 2-bit slots (same codes), row-major
// [n][k/4] bytes.
hipError_t launch_trit5_to_slot2(const uint8_t* trit5, int64_t n, int64_t k, uint8_t* slot2,
                                 hipStream_t stream);
// The 1-bit packing rewritten as 2-bit slots (digit 2b), row-major [n][k/4] bytes.
// count of packed bytes that are not valid encodings of format fmt, added to
// *count (a device int the caller cleared)
hipError_t launch_count_invalid(const uint8_t* packed, int64_t n, int64_t k, int fmt,
                                int32_t* count, hipStream_t stream);
hipError_t launch_bit1_to_slot2(const uint8_t* bit1, int64_t n, int64_t k, uint8_t* slot2,
                                hipStream_t stream);
// Decode GEMV of the 1-bit packing (any m; tokens in launches of at most 16)
hipError_t launch_gemv_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                            int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            hipStream_t stream);
// Prefill GEMM of the 2-bit-slot packing with the weights decoded in
// registers; usable when gemm_slot2_fits(m, n, k).  Its launch plan: `tiles`
// output tiles, tiles [0, t0) computed whole, each later one split along K
// into `splits` parts whose fp32 partial sums need workspace.  row_scale
// (optional): every output of row m is multiplied by row_scale[m].
bool gemm_slot2_fits(int64_t m, int64_t n, int64_t k);
struct Gemm2Plan {
    int64_t tiles, t0;
    int splits;
};
Gemm2Plan gemm_slot2_plan(int64_t m, int64_t n, int64_t k);
int64_t gemm_slot2_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16, void* ws,
                             int64_t ws_bytes, hipStream_t stream, const float* row_scale = nullptr);
// Rotate real-valued weight rows and round them to ternary g128
hipError_t launch_quantize(const float* w, const int8_t* signs, int64_t n, int64_t k,
                           int8_t* codes, uint16_t* scales, hipStream_t stream);
// Prefill products (fp16 or bfloat16 activations) of any packing.  Dense
// trits and 1-bit codes are first rewritten as 2-bit slots into the start of
// the caller's workspace; bfloat16 activations then get their binary16 copy
// and row scales; the K-split partial sums follow, each part at a 256-byte
// boundary.  gemm_workspace_bytes gives the bytes a call needs (0: none);
// gemm_fits whether the shape is supported at all.
bool gemm_fits(int64_t m, int64_t n, int64_t k);
int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int fmt, bool bf16);
hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt,
                       const uint16_t* x, int64_t m, int64_t n, int64_t k,
                       void* y, int y_f16, void* ws, int64_t ws_bytes, hipStream_t stream);
// The product with bfloat16 activations: each row scaled by a power of two
// and converted exactly to binary16, the binary16 product, the power of two
// undone on the outputs
hipError_t launch_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int fmt,
                            const uint16_t* x, int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            void* ws, int64_t ws_bytes, hipStream_t stream);
// Decode chains (tl_linear_chain): plan and sync-buffer sizes, the host-side
// check and encoding of a chain (a tl_status), and the launch.
int64_t chain_plan_bytes(int64_t count);
int64_t chain_sync_bytes(int64_t count);
int chain_encode(const tl_chain_op* ops, int32_t count, void* plan_out);
hipError_t launch_chain(const void* plan, int32_t count, uint32_t* sync, hipStream_t stream);
// Device address and size of the current device's copy of the file-scope
// workspace of tl_gemm_noalloc (looked up once per device; thread-safe).
hipError_t noalloc_scratch(void** out, int64_t* bytes);

}  // namespace tl
