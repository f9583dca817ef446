// Forward kernels: bfloat16 activations, float32 parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_FWD(bf16_f32w, bf16_bits, float, FwdPlans2BW, RowPlans2BW)
}  // namespace rn
