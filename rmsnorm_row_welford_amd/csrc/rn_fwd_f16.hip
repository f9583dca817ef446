// Forward kernels: IEEE binary16 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_FWD(f16, f16_t, f16_t, FwdPlans2B, RowPlans2B)
}  // namespace rn
