// Prefill GEMM (int8 matrix cores).  Filled in by the MFMA kernel; until then every call reports
// "not supported" through the ABI (LB_EUNSUPPORTED), never a substitute computation.
#include "lowbit_internal.h"

namespace lb {

hipError_t launch_gemm(int fmt, const uint8_t *W, int64_t N, int64_t K, float w_scale, const int8_t *Xq,
                       const void *Xscale, int64_t M, float *Y, int32_t *sums, hipStream_t s)
{
    (void)fmt, (void)W, (void)N, (void)K, (void)w_scale, (void)Xq, (void)Xscale, (void)M, (void)Y, (void)sums, (void)s;
    return hipErrorNotSupported;
}

} // namespace lb
