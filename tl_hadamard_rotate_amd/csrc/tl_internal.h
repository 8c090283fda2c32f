// Internal declarations shared by the HIP translation units of libtl.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tl {

constexpr int kBlock = 1024;        // Hadamard block width
constexpr int kGroup = 128;         // weights per binary16 scale
constexpr int kTrit5GroupBytes = 26;

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
// Dense trits at M = 1 with the rotation fused in front (x unrotated; x_rot
// receives the rotated activations); usable when linear_m1_trit5_fits
bool linear_m1_trit5_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear_m1_trit5(const uint8_t* packed, const uint16_t* scales,
                                  const uint16_t* x, const int8_t* signs, uint16_t* x_rot,
                                  int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream);
hipError_t launch_gemv_trit5(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream);
// Library-owned device workspace of `kind` for `stream` on the current
// device, at least `bytes` long (grown with hipMalloc when needed).
enum { kWorkspacePartials = 0, kWorkspaceSlot2 = 1 };
hipError_t workspace(int kind, hipStream_t stream, size_t bytes, void** out);
// The dense trit packing rewritten as 2-bit slots (same codes), row-major
// [n][k/4] bytes.
hipError_t launch_trit5_to_slot2(const uint8_t* trit5, int64_t n, int64_t k, uint8_t* slot2,
                                 hipStream_t stream);
// The 1-bit packing rewritten as 2-bit slots (digit 2b), row-major [n][k/4] bytes.
hipError_t launch_bit1_to_slot2(const uint8_t* bit1, int64_t n, int64_t k, uint8_t* slot2,
                                hipStream_t stream);
// Decode GEMV of the 1-bit packing (any m; tokens in launches of at most 16)
hipError_t launch_gemv_bit1(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                            int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            hipStream_t stream);
// Prefill GEMM of the 2-bit-slot packing with the weights decoded in
// registers; usable when gemm_slot2_fits(m, n, k)
bool gemm_slot2_fits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_slot2(const uint8_t* packed, const uint16_t* scales, const uint16_t* x,
                             int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                             hipStream_t stream);
// Rotate real-valued weight rows and round them to ternary g128
hipError_t launch_quantize(const float* w, const int8_t* signs, int64_t n, int64_t k,
                           int8_t* codes, uint16_t* scales, hipStream_t stream);
// The product with bfloat16 activations: codes as bfloat16 -1/0/+1 on the
// matrix cores, each group's fp32 sums times the binary16 scale
hipError_t launch_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int fmt,
                            const uint16_t* x, int64_t m, int64_t n, int64_t k, void* y, int y_f16,
                            hipStream_t stream);
// Measurement helper: streaming read of `bytes` (a multiple of 16) with `blocks` workgroups
hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* out, int blocks,
                              hipStream_t stream);
hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int fmt,
                       const uint16_t* x, int64_t m, int64_t n, int64_t k,
                       void* y, int y_f16, hipStream_t stream);

}  // namespace tl
