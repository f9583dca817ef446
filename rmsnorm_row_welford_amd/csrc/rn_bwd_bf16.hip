// Backward kernels, bfloat16 storage.
#include "rn_plans.h"

namespace rn {
int bwd_partials_bf16(int64_t N, int H, bool vec, int cus) {
    return bwd_partials_t<bf16_bits, BwdPlansBf16>(N, H, vec, cus);
}
hipError_t launch_bwd_bf16(bool ln, bool fused, const BwdArgs &a, bool vec, int cus,
                          int P, bool colsum, void *dgamma, void *dbeta, hipStream_t s) {
    return launch_bwd_t<bf16_bits, BwdPlansBf16>(ln, fused, a, vec, P, colsum, cus, dgamma, dbeta, s);
}
}  // namespace rn
