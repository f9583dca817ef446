// Forward kernels: binary16 activations, float32 parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_FWD(f16_f32w, f16_t, float, FwdPlans2BW, RowPlans2BW)
}  // namespace rn
