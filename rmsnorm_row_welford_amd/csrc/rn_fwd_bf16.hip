// Forward kernels, bfloat16 storage.
#include "rn_plans.h"

namespace rn {
hipError_t launch_fwd_bf16(int op, const FwdArgs &a, bool vec, int cus,
                           hipStream_t s) {
    return launch_fwd_t<bf16_bits, FwdPlansBf16>(op, a, vec, cus, s);
}
}  // namespace rn
