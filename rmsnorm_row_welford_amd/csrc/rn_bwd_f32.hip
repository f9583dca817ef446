// Backward kernels, float32 storage.
#include "rn_plans.h"

namespace rn {
int bwd_partials_f32(int64_t N, int H, bool vec, int cus) {
    return bwd_partials_t<float, BwdPlansF32>(N, H, vec, cus);
}
hipError_t launch_bwd_f32(bool ln, bool fused, const BwdArgs &a, bool vec, int cus,
                          int P, bool colsum, void *dgamma, void *dbeta, hipStream_t s) {
    return launch_bwd_t<float, BwdPlansF32>(ln, fused, a, vec, P, colsum, cus, dgamma, dbeta, s);
}
}  // namespace rn
