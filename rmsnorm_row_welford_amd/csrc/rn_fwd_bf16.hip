// Forward kernels: bfloat16 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_FWD(bf16, bf16_bits, bf16_bits, FwdPlans2B, RowPlans2B)
}  // namespace rn
