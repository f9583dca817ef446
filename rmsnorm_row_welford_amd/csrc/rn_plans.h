// Plan tables: which team shape serves a row of H elements.
//
// Forward rows live in registers (E = VEC*CPL floats per lane plus gamma and
// beta), backward rows need x_hat, g and two accumulators per element, so
// the backward keeps E <= 16 and widens the team instead.  Rows whose H,
// strides or base addresses are not multiples of 16 bytes take the
// element-wise (VEC = 1) plans.
#pragma once

#include "rn_kernels.h"

namespace rn {

// Walk a list of plans and run `f.template operator()<P>()` on the first
// plan whose span covers H.
template <class... Ps> struct PlanList {};

template <class F>
hipError_t pick_plan(PlanList<>, int, F &&) {
    return hipErrorInvalidValue;
}
template <class P, class... Ps, class F>
hipError_t pick_plan(PlanList<P, Ps...>, int H, F &&f) {
    if (H <= P::SPAN) return f.template operator()<P>();
    return pick_plan(PlanList<Ps...>{}, H, f);
}

template <class F>
int pick_plan_int(PlanList<>, int, F &&) { return -1; }
template <class P, class... Ps, class F>
int pick_plan_int(PlanList<P, Ps...>, int H, F &&f) {
    if (H <= P::SPAN) return f.template operator()<P>();
    return pick_plan_int(PlanList<Ps...>{}, H, f);
}

// Plans for 2-byte activations (bf16, fp16).  Those for the benchmarked
// row lengths can be overridden at build time (-DRN_FWD_BF16_1024=... etc.)
// to sweep team shapes.
// Forward plans that run one workgroup per row group (several fit per CU)
// do not prefetch (PF = false): the registers would go unused.
#ifndef RN_FWD_BF16_1024
#define RN_FWD_BF16_1024 Plan<8, 2, 1, 4, false>
#endif
#ifndef RN_FWD_BF16_2048
#define RN_FWD_BF16_2048 Plan<8, 4, 1, 4, false>
#endif
#ifndef RN_FWD_BF16_4096
#define RN_FWD_BF16_4096 Plan<8, 2, 4, 1, false>
#endif
#ifndef RN_FWD_BF16_16384
#define RN_FWD_BF16_16384 Plan<8, 2, 16, 1>
#endif
#ifndef RN_BWD_BF16_1024
#define RN_BWD_BF16_1024 Plan<8, 2, 1, 8>
#endif
#ifndef RN_BWD_BF16_2048
#define RN_BWD_BF16_2048 Plan<8, 2, 2, 4>
#endif
#ifndef RN_BWD_BF16_16384
#define RN_BWD_BF16_16384 Plan<8, 2, 16, 1>
#endif

// ------------------------------------------------------------- forward --
using FwdPlans2B = PlanList<Plan<8, 1, 1, 4, false>,     //   512
                              RN_FWD_BF16_1024,            //  1024
                              RN_FWD_BF16_2048,            //  2048
                              RN_FWD_BF16_4096,            //  4096
                              Plan<8, 2, 8, 1, false>,     //  8192
                              RN_FWD_BF16_16384>;          // 16384
using FwdPlansF32 = PlanList<Plan<4, 1, 1, 4, false>,      //   256
                             Plan<4, 2, 1, 4, false>,      //   512
                             Plan<4, 4, 1, 4, false>,      //  1024
                             Plan<4, 4, 2, 2, false>,      //  2048
                             Plan<4, 4, 4, 1, false>,      //  4096
                             Plan<4, 4, 8, 1, false>,      //  8192
                             Plan<4, 4, 16, 1>>;           // 16384
using FwdPlansScalar = PlanList<Plan<1, 1, 1, 4>,   //    64
                                Plan<1, 4, 1, 4>,   //   256
                                Plan<1, 4, 4, 1>,   //  1024
                                Plan<1, 4, 16, 1>,  //  4096
                                Plan<1, 8, 16, 1>>; //  8192

// ------------------------------------------------------------ backward --
using BwdPlans2B = PlanList<Plan<8, 1, 1, 8>,     //   512
                              RN_BWD_BF16_1024,     //  1024
                              RN_BWD_BF16_2048,     //  2048
                              Plan<8, 2, 4, 2>,     //  4096
                              Plan<8, 2, 8, 1>,     //  8192
                              RN_BWD_BF16_16384>;   // 16384
// float32 rows of 16 elements per lane are too wide to double-buffer.
using BwdPlansF32 = PlanList<Plan<4, 1, 1, 8>,             //   256
                             Plan<4, 2, 1, 8>,             //   512
                             Plan<4, 4, 1, 8, false>,      //  1024
                             Plan<4, 4, 2, 4, false>,      //  2048
                             Plan<4, 4, 4, 2, false>,      //  4096
                             Plan<4, 4, 8, 1, false>,      //  8192
                             Plan<4, 4, 16, 1, false>>;    // 16384
using BwdPlansScalar = PlanList<Plan<1, 1, 1, 8>,   //    64
                                Plan<1, 4, 1, 8>,   //   256
                                Plan<1, 4, 4, 2>,   //  1024
                                Plan<1, 4, 16, 1>,  //  4096
                                Plan<1, 8, 16, 1>>; //  8192

template <class T, class W, class VecPlans>
hipError_t launch_fwd_t(int op, const FwdArgs &a, bool vec, int cus,
                        hipStream_t s) {
    auto f = [&]<class P>() { return launch_fwd_op<T, W, P>(op, a, cus, s); };
    return vec ? pick_plan(VecPlans{}, a.H, f)
               : pick_plan(FwdPlansScalar{}, a.H, f);
}

template <class T, class W, class VecPlans>
int bwd_partials_t(int64_t N, int H, bool vec, int cus) {
    auto f = [&]<class P>() { return bwd_grid<T, W, P>(N, H, cus); };
    return vec ? pick_plan_int(VecPlans{}, H, f)
               : pick_plan_int(BwdPlansScalar{}, H, f);
}

template <class T, class W, class VecPlans>
hipError_t launch_bwd_t(bool ln, bool fused, const BwdArgs &a, bool vec, int P,
                        bool colsum, int cus, void *dg, void *db, hipStream_t s) {
    auto f = [&]<class Pl>() {
        return launch_bwd_plan<T, W, Pl>(ln, fused, a, P, colsum, cus, dg, db, s);
    };
    return vec ? pick_plan(VecPlans{}, a.H, f)
               : pick_plan(BwdPlansScalar{}, a.H, f);
}

// Body of the translation units: the three entry points for storage pair
// S = (T activations, W parameters) with the given vector plan lists.
#define RN_DEFINE_FWD(S, T, W, PLANS)                                              \
    hipError_t launch_fwd_##S(int op, const FwdArgs &a, bool vec, int cus,         \
                              hipStream_t s) {                                     \
        return launch_fwd_t<T, W, PLANS>(op, a, vec, cus, s);                      \
    }
#define RN_DEFINE_BWD(S, T, W, PLANS)                                              \
    int bwd_partials_##S(int64_t N, int H, bool vec, int cus) {                    \
        return bwd_partials_t<T, W, PLANS>(N, H, vec, cus);                        \
    }                                                                              \
    hipError_t launch_bwd_##S(bool ln, bool fused, const BwdArgs &a, bool vec,     \
                              int cus, int P, bool colsum, void *dgamma,           \
                              void *dbeta, hipStream_t s) {                        \
        return launch_bwd_t<T, W, PLANS>(ln, fused, a, vec, P, colsum, cus, dgamma, \
                                         dbeta, s);                                \
    }

}  // namespace rn
