// Backward kernels: IEEE binary16 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_BWD(f16, f16_t, f16_t, BwdPlans2B)
}  // namespace rn
