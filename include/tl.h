/*
 * tl.h — C ABI of the ternary g128 linear-layer library for MI355X (gfx950).
 *
 * The layer computes  y = dequant(codes, scales) · R(x)  where
 *   - codes are ternary weights in {-1, 0, +1} with one binary16 scale per 128
 *     consecutive weights of a row ("ternary g128"); source: page "A 27-billion
 *     model that fits in 8.6 GB" (news.ditty.ir), paragraph 2, and page
 *     "Ternary Bonsai 2 27B: 27B-модель в 5,9 ГБ" (ai4coding.ru), section
 *     "Что такое тернарная модель";
 *   - R is the signed block-Hadamard rotation over 1024-wide blocks that was
 *     folded into the weights and must be applied to the activations at run
 *     time; source: the Persian page, paragraphs 2 and 3, and page "OpenBonsai"
 *     (openbonsai.org), section "How it works", step 1;
 *   - the codes are stored in one of two byte packings of the same weights, a
 *     dense one with 5 trits per byte and one with a 2-bit slot per weight;
 *     source: the Persian page, paragraph 5.
 *
 * Conventions shared by every call
 *   - All tensors are dense row-major device buffers owned by the caller; the
 *     library never allocates, frees or retains device memory (outside the
 *     opt-in debug checks below).  The prefill products take a caller-owned
 *     workspace (tl_gemm_workspace_bytes).
 *   - binary16 data is passed as uint16_t (bit patterns).
 *   - Every call validates its arguments first.  On a validation failure it
 *     returns the status and launches nothing, so outputs are untouched.
 *   - On success the work is enqueued on `stream` (0 = the null stream) and the
 *     call returns TL_OK without synchronising.  A launch failure returns
 *     TL_ERR_LAUNCH and tl_last_error() gives the HIP error text (per thread).
 *   - The library keeps no state between calls apart from that per-thread
 *     error text and, per device, the compute-unit count and the kernels' LDS
 *     limits, looked up on first use; calls from several threads are safe.
 *   - Debug checks: with the environment variable TL_DEBUG=1, tl_unpack,
 *     tl_gemv, tl_gemm, tl_gemm_bf16 and tl_linear first count the packed
 *     bytes that are not valid encodings (see Formats) on the device, wait
 *     for the count on `stream`, and return TL_ERR_DATA (count in
 *     tl_last_error()) without launching anything else when there is any.
 *     This mode synchronises, allocates one small device buffer per GPU on
 *     first use and serialises the checks of concurrent calls; it is skipped
 *     while `stream` is being captured, and tl_gemm_noalloc and
 *     tl_linear_chain never check.
 *
 * Formats (bit-exact; defined here, since the pages give no byte layout)
 *   digit d = code + 1, in {0, 1, 2}.
 *   TL_FMT_TRIT5: each row holds K/128 groups of 26 bytes (row stride 26*K/128
 *     bytes).  Byte j < 25 of a group = sum_{i<5} d[5j+i] * 3^i (values 0..242,
 *     first digit least significant).  Byte 25 = d[125] + 3 d[126] + 9 d[127]
 *     + 27 + 81: the two pad digits are 1 (code 0), values 108..134.
 *     1.625 code bits + 0.125 scale bits = 1.75 bits per weight.
 *   TL_FMT_SLOT2: each row holds K/4 bytes; bits 2i..2i+1 of byte j hold
 *     d[4j+i].  2.125 bits per weight with the scales.
 *   TL_FMT_BIT1: codes -1 and +1 only, one bit b = (code + 1) / 2 each: each
 *     row holds K/8 bytes and bit i of byte j holds b[8j+i].  1.125 bits per
 *     weight with the scales (page "How Prism ML Squeezed a 27B Model Into
 *     3.9 GB", list "Two formats ship today").
 *   Packed bytes that are not valid encodings (a 2-bit slot holding 3, a
 *     dense-trit byte above 242, a group's last byte whose pad digits are not
 *     1) give unspecified results in every call that reads packed codes (the
 *     kernels stay within their buffers).  tl_pack never writes such bytes; it
 *     counts the invalid codes it was given in bad_count.
 *   Scales: binary16 [N, K/128]; weight (n, k) = code * scales[n, k/128].
 *   Signs: int8 [K] of +1/-1; block b of the rotation uses signs[1024b .. +1023].
 */
#ifndef TL_H
#define TL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define TL_API __attribute__((visibility("default")))
#else
#define TL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TL_OK = 0,
    TL_ERR_NULL = 1,     /* a required pointer is NULL                          */
    TL_ERR_SHAPE = 2,    /* a size is out of range (see each call)             */
    TL_ERR_FORMAT = 3,   /* unknown packing format                             */
    TL_ERR_ALIGN = 4,    /* a pointer is not 16-byte aligned                   */
    TL_ERR_ALIAS = 5,    /* an output overlaps an input it must not overlap    */
    TL_ERR_LAUNCH = 6,   /* the HIP launch failed; see tl_last_error()         */
    TL_ERR_DTYPE = 7,    /* unknown output dtype                               */
    TL_ERR_WORKSPACE = 8, /* workspace missing or smaller than the call needs  */
    TL_ERR_DATA = 9      /* invalid packed bytes found (only with TL_DEBUG=1)  */
} tl_status;

enum { TL_FMT_TRIT5 = 0, TL_FMT_SLOT2 = 1, TL_FMT_BIT1 = 2 };
enum { TL_F32 = 0, TL_F16 = 1 };

#define TL_BLOCK 1024      /* Hadamard block width                 */
#define TL_GROUP 128       /* weights per scale                    */
#define TL_MAX_K (1 << 20) /* largest K any call accepts           */

/* Bytes of the packed code array for an N x K weight in format `fmt`
 * (scales not included).  Host only.  Returns -1 when N < 1, K < 128,
 * K % 128 != 0 or fmt is unknown. */
TL_API int64_t tl_packed_bytes(int64_t N, int64_t K, int32_t fmt);

/* Pack ternary codes.  codes: int8 [N, K] (device); packed: uint8 of
 * tl_packed_bytes(N, K, fmt) bytes (device).  Requires 1 <= N <= 2^24,
 * K >= 128, K % 128 == 0, K <= TL_MAX_K, N * K <= 2^36.  codes and packed
 * must be 16-byte aligned, bad_count 4-byte aligned.  A code outside {-1, 0, 1} is packed as 0
 * and counted; with TL_FMT_BIT1 every code other than -1 and +1 is packed as +1
 * and counted: when bad_count (device int32, may be NULL) is given, the
 * number of such codes is ADDED to *bad_count (the caller clears it).
 * packed must not overlap codes.  Bit-exact with the format above. */
TL_API tl_status tl_pack(const int8_t* codes, int64_t N, int64_t K, int32_t fmt,
                  uint8_t* packed, int32_t* bad_count, hipStream_t stream);

/* Unpack to int8 codes [N, K] (device).  Same shape rules as tl_pack.
 * Bytes that are not valid encodings give unspecified codes in {-1, 0, 1}. */
TL_API tl_status tl_unpack(const uint8_t* packed, int64_t N, int64_t K, int32_t fmt,
                    int8_t* codes, hipStream_t stream);

/* Signed block-Hadamard rotation of the rows of x:
 *   x_rot[m, 1024b + i] = (1/32) sum_j H[i, j] signs[1024b + j] x[m, 1024b + j]
 * with H the Sylvester Hadamard matrix of order 1024 (H[i,j] = (-1)^popcount(i&j)).
 * x, x_rot: binary16 [M, K]; signs: int8 [K].  Computed in fp32, rounded to
 * binary16 to nearest even.  Requires 1 <= M <= 2^24, K >= 1024,
 * K % 1024 == 0, K <= TL_MAX_K, M * K <= 2^36.  A negative sign byte means -1,
 * any other value +1.  x_rot may equal x (in place) but must not otherwise
 * overlap x or signs.  Source: the Persian page, paragraphs 2 and 3. */
TL_API tl_status tl_hadamard_rotate(const uint16_t* x, const int8_t* signs, int64_t M, int64_t K,
                             uint16_t* x_rot, hipStream_t stream);

/* Ternary linear on already rotated activations (decode shapes):
 *   y[m, n] = sum_k x_rot[m, k] * code[n, k] * scales[n, k/128]
 * packed: [N, ...] in format fmt; scales: binary16 [N, K/128]; x_rot: binary16
 * [M, K]; y: [M, N] of y_dtype (TL_F32, or TL_F16 rounded to nearest even).
 * Products are exact, sums in fp32, and the result does not depend on the
 * launch (bitwise deterministic).  Requires 1 <= M, N <= 2^24, K >= 1024,
 * K % 1024 == 0, K <= TL_MAX_K, and M*K, N*K, M*N <= 2^36.  Tuned for
 * M <= 16; any M is accepted.  y must
 * not overlap any input.  Multiply-accumulate with ternary weights is
 * additions and subtractions (ai4coding.ru page, section "Что такое тернарная
 * модель"). */
TL_API tl_status tl_gemv(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                  const uint16_t* x_rot, int64_t M, int64_t N, int64_t K,
                  void* y, int32_t y_dtype, hipStream_t stream);

/* Bytes of device workspace that tl_gemm and tl_linear need for this shape
 * and format (0: none; tl_linear at M < 64 needs none).  Host only; it
 * depends on the compute-unit count of the current device.  Returns -1 when
 * the shape or format is not accepted (tl_gemm's rules).  The workspace
 * holds, for dense trits and 1-bit codes, the weights rewritten as 2-bit
 * slots (N * K/4 bytes, rounded up to 256), then, when output tiles are split
 * along K, their fp32 partial sums (at most 64 MiB). */
TL_API int64_t tl_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t fmt);

/* The same for tl_gemm_bf16: the rewrite as above, then the binary16 copy of
 * the activations (M * K * 2 bytes) and M fp32 row factors (each rounded up
 * to 256 bytes), then the K-split partial sums. */
TL_API int64_t tl_gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t fmt);

/* Launch plan of tl_gemm for this shape (host only, for tests and tuning):
 * out[0] = output tiles of 256 x 256, out[1] = tiles computed whole, out[2] =
 * parts along K of each remaining tile.  Returns TL_OK, TL_ERR_NULL or
 * TL_ERR_SHAPE (tl_gemm's shape rules). */
TL_API tl_status tl_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t* out);

/* Same operation and argument rules as tl_gemv, tuned for prefill (M >= 64):
 * weight tiles are expanded to exact binary16 (code * scale) on chip and fed
 * to fp16 matrix-core instructions with fp32 accumulation.  Prompt processing
 * is where the pages place the practical bottleneck on slower chips (Persian
 * page, paragraph 4).
 * Output tiles that would leave most of the GPU idle in a last partial round
 * are split along K; their fp32 partial sums go to the workspace and a second
 * kernel adds them in a fixed order (results do not depend on scheduling).
 * Dense trits and 1-bit codes are first rewritten as 2-bit slots (same codes)
 * into the workspace, then multiplied the same way.
 * workspace: caller-owned device memory of workspace_bytes >=
 * tl_gemm_workspace_bytes(M, N, K, fmt) bytes (may be NULL when that is 0),
 * 16-byte aligned, overlapping no argument; its contents on entry do not
 * matter, and calls that may run at the same time need separate workspaces.
 * Too small: TL_ERR_WORKSPACE.  Additionally requires M * K < 2^31 and
 * N * K / 4 < 2^32 (TL_ERR_SHAPE). */
TL_API tl_status tl_gemm(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                  const uint16_t* x_rot, int64_t M, int64_t N, int64_t K,
                  void* y, int32_t y_dtype, void* workspace, int64_t workspace_bytes,
                  hipStream_t stream);

/* tl_gemm without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same operation, rules, kernels, launch plan and
 * results (bit for bit) as tl_gemm; it calls no allocator.  Its workspace is
 * a file-scope device array of TL_GEMM_NOALLOC_MAX_WORKSPACE bytes (96 MiB)
 * that every GPU the library runs on holds until the process ends; a shape
 * whose tl_gemm_workspace_bytes exceeds it returns TL_ERR_WORKSPACE (dense
 * trits and 1-bit codes need N * K / 4 bytes for their rewrite, so N * K up
 * to 2^27 weights).  All calls on one GPU share that array: calls that may
 * run at the same time on one GPU (other streams, other threads) race and
 * must not be issued; calls in order on one stream are safe. */
#define TL_GEMM_NOALLOC_MAX_WORKSPACE (96 << 20)
TL_API tl_status tl_gemm_noalloc(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                                 const uint16_t* x_rot, int64_t M, int64_t N, int64_t K,
                                 void* y, int32_t y_dtype, hipStream_t stream);

/* The whole layer on unrotated activations:
 *   x_rot = R(x)  (as tl_hadamard_rotate),   y = dequant(codes, scales) . x_rot
 * i.e. y[m, n] = sum_k R(x)[m, k] * code[n, k] * scales[n, k/128]: the
 * runtime rotation of the activations that the folded weights require (the
 * Persian page, paragraphs 2 and 3) followed by the ternary product.
 * x: binary16 [M, K], not rotated; signs: int8 [K]; x_rot: binary16 [M, K],
 * caller-owned, receives R(x) (rounded to binary16 as tl_hadamard_rotate
 * does); y as for tl_gemv.  Shape, format, dtype and alignment rules as
 * tl_gemv (x in place of x_rot); x_rot must not overlap x, signs, packed,
 * scales or y, and y must not overlap any input.  At M = 1 with
 * TL_FMT_SLOT2 (K <= 26624) or TL_FMT_TRIT5 (K <= 18432, and up to 22528 for
 * most N) the rotation runs inside the GEMV kernel: one launch, the rotated
 * activations never make a round trip through memory before use (x_rot is
 * still written).  Otherwise: tl_hadamard_rotate, then tl_gemv (M < 64) or
 * tl_gemm (M >= 64, with the workspace as tl_gemm; unused below 64).
 * Linears that read the same input (q, k, v; gate, up) share its rotation:
 * the signs belong to the input, so their packed rows and scales can be
 * concatenated along N (row-major, so plain concatenation) and run as one
 * call, which rotates once and launches once. */
TL_API tl_status tl_linear(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                    const uint16_t* x, const int8_t* signs, int64_t M, int64_t N, int64_t K,
                    uint16_t* x_rot, void* y, int32_t y_dtype, void* workspace,
                    int64_t workspace_bytes, hipStream_t stream);

/* One linear of a decode chain (tl_linear_chain): the arguments of tl_linear
 * at M = 1.  packed: TL_FMT_SLOT2 codes [N, K/4]; scales [N, K/128]; x: the
 * unrotated binary16 input [K], either ready when the chain starts or lying
 * within the binary16 y of an earlier linear of the chain; signs [K]; x_rot: [K]
 * binary16 receiving R(x), or NULL; y: [N] of y_dtype. */
typedef struct {
    const uint8_t* packed;
    const uint16_t* scales;
    const uint16_t* x;
    const int8_t* signs;
    uint16_t* x_rot;
    void* y;
    int64_t N;
    int64_t K;
    int32_t fmt;
    int32_t y_dtype;
} tl_chain_op;

/* Bytes of the encoded plan and of the sync buffer of a chain of `count`
 * linears (1 <= count <= 65536; -1 otherwise).  Host only. */
TL_API int64_t tl_chain_plan_bytes(int32_t count);
TL_API int64_t tl_chain_sync_bytes(int32_t count);

/* Check a chain and encode its plan into `plan` (HOST memory of plan_bytes
 * >= tl_chain_plan_bytes(count) bytes), which the caller copies to device
 * memory once and may launch any number of times.  Rules: fmt TL_FMT_SLOT2;
 * 1 <= N <= 2^24; K % 1024 == 0, 1024 <= K <= 32768, with each workgroup's
 * share of the rows (ceil(N / CUs)) times K/1024 at most 2048 and its LDS
 * within one CU (TL_ERR_SHAPE); every pointer 16-byte aligned.  An output (y,
 * x_rot) may overlap nothing else of the chain except that the x of a later
 * linear may lie within a binary16 y, and that linear then waits for the whole
 * y to be written (else TL_ERR_ALIAS).  The plan records the
 * compute-unit count of the current device and is valid only there.  Bytes
 * 12..15 of the plan (uint32) hold the number of polls after which a wait for
 * an input gives up (set by the encoder; a smaller value only makes a failure
 * show sooner). */
TL_API tl_status tl_chain_encode(const tl_chain_op* ops, int32_t count, void* plan,
                                 int64_t plan_bytes);

/* Run an encoded chain in one launch: each linear is tl_linear at M = 1 (the
 * same results, bit for bit), in order, with the next linear's weight stream
 * starting before the current one has finished, so the stream does not stop
 * at linear boundaries (the rotation still runs on every linear's input:
 * Persian page, paragraph 3).  plan: device copy of tl_chain_encode's
 * output; sync: device uint32 [tl_chain_sync_bytes(count) / 4], all zero
 * before the first call, not overlapping plan; every completed call leaves it
 * as it found it except word count + 1, the error word, which a failure sets
 * (first failure kept) and only the caller clears: 1 = the plan does not
 * match count or the device, 2 + i = linear i's wait for its input gave up
 * (its input was not complete within the plan's poll limit: the GPU must not
 * be shared with other work while a chain with such waits runs).  After a
 * failure the outputs are unspecified.  Calls sharing a sync buffer must not
 * run at the same time. */
TL_API tl_status tl_linear_chain(const void* plan, int32_t count, uint32_t* sync,
                                 hipStream_t stream);

/* The prefill product with bfloat16 rotated activations:
 *   y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x_rot[m, k]
 * for models whose activations are bfloat16.  Each row of x_rot is scaled by
 * the power of two that brings its largest |x| into [2^14, 2^15) and
 * converted to binary16, which is exact for a bfloat16 number (8 significant
 * bits) unless it is below 2^-17 of that range; the product then runs as
 * tl_gemm's (exact binary16 code * scale, fp32 sums) and the outputs are
 * multiplied back by the power of two.  x_rot: bfloat16 [M, K] passed as
 * uint16 bits; workspace: at least tl_gemm_bf16_workspace_bytes; every other
 * argument, rule and error as tl_gemm. */
TL_API tl_status tl_gemm_bf16(const uint8_t* packed, const uint16_t* scales, int32_t fmt,
                              const uint16_t* x_rot, int64_t M, int64_t N, int64_t K, void* y,
                              int32_t y_dtype, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);

/* Quantise real-valued weight rows to ternary g128, the rotation folded in
 * (page "OpenBonsai", section "How it works", steps 1 and 2: rotate with the
 * signed Hadamard transform, then round to -1, 0, +1 with one scale per 128;
 * the page rounds by GPTQ on calibration data, this call by round to nearest;
 * page "A 27-billion model that fits in 8.6 GB", paragraph 2: FP16 scales).
 *   w'  = R(w) row by row (the map tl_hadamard_rotate applies, fp32 here);
 *   S   = the binary16 nearest to the mean of |w'| over each group of 128;
 *   c   = rint(w' / S) clipped to [-1, 1], ties to even (|w'| = S/2 gives 0),
 *         c = 0 where S = 0.
 * w: fp32 [N, K]; signs: int8 [K] (negative = -1); codes: int8 [N, K];
 * scales: binary16 [N, K/128]; all device memory, 16-byte aligned.
 * 1 <= N <= 2^24, K % 1024 == 0, 1024 <= K <= TL_MAX_K, N * K <= 2^36.
 * codes and scales must not overlap each other, w or signs.  The result is
 * bitwise reproducible; codes then go to tl_pack. */
TL_API tl_status tl_quantize(const float* w, const int8_t* signs, int64_t N, int64_t K,
                             int8_t* codes, uint16_t* scales, hipStream_t stream);

/* Static name of a status code ("TL_OK", ...). */
TL_API const char* tl_status_str(tl_status status);

/* Text of the last TL_ERR_LAUNCH on the calling thread ("" if none). */
TL_API const char* tl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TL_H */
