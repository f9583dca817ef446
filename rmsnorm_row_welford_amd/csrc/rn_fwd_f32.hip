// Forward kernels: float32 activations and parameters.
#include "rn_plans.h"

namespace rn {
RN_DEFINE_FWD(f32, float, float, FwdPlansF32)
}  // namespace rn
