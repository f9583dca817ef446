// Forward kernels, float32 storage.
#include "rn_plans.h"

namespace rn {
hipError_t launch_fwd_f32(int op, const FwdArgs &a, bool vec, int cus,
                          hipStream_t s) {
    return launch_fwd_t<float, FwdPlansF32>(op, a, vec, cus, s);
}
}  // namespace rn
