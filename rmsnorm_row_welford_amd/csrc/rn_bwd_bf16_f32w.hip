// Backward kernels: bfloat16 activations, float32 parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_BWD(bf16_f32w, bf16_bits, float, BwdPlans2B)
}  // namespace rn
