// Decode products y[m, n] = sum_g S[n, g] * sum_{k in g} code[n, k] * x[m, k]
// (tl_gemv): the kernel for each packing and token count.
#include "tl_internal.h"

namespace tl {

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int fmt, const uint16_t* x,
                       int64_t m, int64_t n, int64_t k, void* y, int y_f16, hipStream_t stream) {
    switch (fmt) {
        case 0: return launch_gemv_trit5(packed, scales, x, m, n, k, y, y_f16, stream);
        case 1:
            if (gemv_m1_slot2_fits(m, n, k))
                return launch_gemv_m1_slot2(packed, scales, x, n, k, y, y_f16, stream);
            if (gemv_mt_slot2_fits(m, n, k))
                return launch_gemv_mt_slot2(packed, scales, x, m, n, k, y, y_f16, stream);
            return launch_gemv_slot2(packed, scales, x, m, n, k, y, y_f16, stream);
        case 2:
            if (gemv_m1_bit1_fits(m, n, k))
                return launch_gemv_m1_bit1(packed, scales, x, n, k, y, y_f16, stream);
            if (gemv_mt_bit1_fits(m, n, k))
                return launch_gemv_mt_bit1(packed, scales, x, m, n, k, y, y_f16, stream);
            return launch_gemv_bit1(packed, scales, x, m, n, k, y, y_f16, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tl
