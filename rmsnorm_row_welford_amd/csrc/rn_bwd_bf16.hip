// Backward kernels: bfloat16 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_BWD(bf16, bf16_bits, bf16_bits, BwdPlans2B)
}  // namespace rn
