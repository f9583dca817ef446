// Backward kernels: float32 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_BWD(f32, float, float, BwdPlansF32)
}  // namespace rn
