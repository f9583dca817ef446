// Plan tables: which team shape serves a row of H elements.
//
// Forward rows live in registers (E = VEC*CPL floats per lane plus gamma and
// beta), backward rows need x_hat, g and two accumulators per element, so
// the backward keeps E <= 16 and widens the team instead.  Rows whose H,
// strides or base addresses are not multiples of 16 bytes take the
// element-wise (VEC = 1) plans.
#pragma once

#include <initializer_list>

#include "rn_kernels.h"
#include "rn_long.h"
#include "rn_seg.h"

namespace rn {

// ------------------------------------------------ several rows per wave --
// Rows of at most SEG*VEC*CPL elements: SEG lanes per row (64: a whole
// wave), 64/SEG rows per wave, CPL chunks per lane, WPG waves per
// workgroup, IT row groups of a wave in flight in the forward (the backward
// forms take CPL = 1, SEG <= 32).  Row strides too large for 32-bit group
// offsets fall back to one row per wave.
template <int VEC_, int SEG_, int WPG_, int IT_, int CPL_ = 1>
struct SegPlan {
    static constexpr int VEC = VEC_, SEG = SEG_, WPG = WPG_, IT = IT_, CPL = CPL_;
    static constexpr int RPW = 64 / SEG_;
    static constexpr int SPAN = SEG_ * VEC_ * CPL_;
    static constexpr int THREADS = 64 * WPG_;
    using Fallback = Plan<VEC_, CPL_, 1, 4, false>;
};

inline bool seg_fits(int rpw, int e, std::initializer_list<int64_t> lds) {
    for (int64_t ld : lds)
        if (ld * e * rpw >= ((int64_t)1 << 31)) return false;
    return true;
}

template <class T, class W, class P, int OP>
hipError_t launch_fwd_seg(const FwdArgs &a, hipStream_t s) {
    constexpr int rows = P::WPG * P::RPW * P::IT;
    const int64_t grid = (a.N + rows - 1) / rows;
    // LayerNorm rows that fill the span exactly need no masking selects
    if constexpr (OP == OP_LN) {
        if (a.H == P::SPAN) {
            hipLaunchKernelGGL(
                (fwd_seg_kernel<T, W, P::VEC, P::SEG, P::CPL, P::WPG, P::IT, OP, true>),
                dim3((unsigned)grid), dim3(P::THREADS), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fwd_seg_kernel<T, W, P::VEC, P::SEG, P::CPL, P::WPG, P::IT, OP>),
                       dim3((unsigned)grid), dim3(P::THREADS), 0, s, a);
    return hipGetLastError();
}

template <class T, class W, class P>
hipError_t launch_fwd_any(int op, const FwdArgs &a, int cus, hipStream_t s) {
    if constexpr (P::SEG > 0) {
        if (seg_fits(P::RPW, (int)sizeof(T), {a.ldx, a.ldr, a.ldy, a.ldh})) {
            switch (op) {
            case OP_LN: return launch_fwd_seg<T, W, P, OP_LN>(a, s);
            case OP_RMS: return launch_fwd_seg<T, W, P, OP_RMS>(a, s);
            default: return launch_fwd_seg<T, W, P, OP_FUSED>(a, s);
            }
        }
        return launch_fwd_op<T, W, typename P::Fallback>(op, a, cus, s);
    } else {
        return launch_fwd_op<T, W, P>(op, a, cus, s);
    }
}

// Kernel 1's workgroup count (= partial rows) of a several-rows-per-wave
// plan; its one-row-per-wave fallback runs with the same count.
template <class T, class W, class P>
int bwd_grid_any(int64_t N, int H, int cus) {
    if constexpr (P::SEG > 0) {
        constexpr auto k = bwd1_seg_kernel<T, W, P::VEC, P::SEG, P::WPG, true, false>;
        if (N <= (int64_t)P::RPW * P::WPG * RN_BWD_DECODE_ROWS) return N > 0 ? 1 : 0;
        const int per_cu = RN_BWD_PER_CU > 0 ? RN_BWD_PER_CU
                                             : resident_per_cu<k>(P::THREADS, 0);
        const int64_t groups = (N + P::RPW * P::WPG - 1) / (P::RPW * P::WPG);
        const int64_t cap = (int64_t)(per_cu < 1 ? 1 : per_cu) * cus;
        return (int)(groups < cap ? groups : cap);
    } else {
        return bwd_grid<T, W, P>(N, H, cus);
    }
}

template <class T, class W, class P, bool LN, bool ADD>
hipError_t launch_bwd_seg(const BwdArgs &a, int P_, void *dg, void *db, hipStream_t s) {
    if (P_ == 1) {
        // one workgroup holds every row: kernel 1 writes dgamma/dbeta itself
        hipLaunchKernelGGL((bwd1_seg_kernel<T, W, P::VEC, P::SEG, P::WPG, LN, ADD, true>),
                           dim3(1), dim3(P::THREADS), 0, s, a);
        return hipGetLastError();
    }
    if (P_ > 0) {
        hipLaunchKernelGGL((bwd1_seg_kernel<T, W, P::VEC, P::SEG, P::WPG, LN, ADD>),
                           dim3(P_), dim3(P::THREADS), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_bwd2<W>(a.part, P_, a.H, LN, dg, db, s);
}

template <class T, class W, class P>
hipError_t launch_bwd_any(bool ln, bool fused, const BwdArgs &a, int P_, bool colsum,
                          int cus, void *dg, void *db, hipStream_t s) {
    if constexpr (P::SEG > 0) {
        if (!colsum && seg_fits(P::RPW, (int)sizeof(T),
                                {a.lddy, a.ldx, a.lddx, a.ldadd, a.lddx2})) {
            if (ln) return launch_bwd_seg<T, W, P, true, false>(a, P_, dg, db, s);
            if (fused) return launch_bwd_seg<T, W, P, false, true>(a, P_, dg, db, s);
            return launch_bwd_seg<T, W, P, false, false>(a, P_, dg, db, s);
        }
        return launch_bwd_plan<T, W, typename P::Fallback>(ln, fused, a, P_, colsum, cus,
                                                           dg, db, s);
    } else {
        return launch_bwd_plan<T, W, P>(ln, fused, a, P_, colsum, cus, dg, db, s);
    }
}

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
// do not prefetch (PF = false): the registers would go unused.  Rows of
// 1-4 KiB run one row per wave with two rows of each wave in flight (a
// whole-wave SegPlan; four 4 KiB rows need too many registers, so one).
#ifndef RN_FWD_BF16_512
#define RN_FWD_BF16_512 SegPlan<8, 64, 4, 2, 1>
#endif
#ifndef RN_FWD_BF16_1024
#define RN_FWD_BF16_1024 SegPlan<8, 64, 4, 2, 2>
#endif
#ifndef RN_FWD_BF16_2048
#define RN_FWD_BF16_2048 SegPlan<8, 64, 4, 1, 4>
#endif
// Rows of 4096 and 8192: LayerNorm and RMSNorm run one 1024-thread
// workgroup per CU (teams of 4 or 8 waves) prefetching their next rows,
// which holds the parameters in registers for all the rows; the fused op
// (twice the row registers) and inputs of fewer than 4 rows per CU (the
// few-row, latency-bound regime) run one small workgroup per row group
// instead (the RowPlans lists).  Measured: at 2048-8192 x 4096 the
// persistent plans are 1-2 us faster for LN/RMS and 4.5 us slower for the
// fused op at 32768 x 4096; at 1-64 rows of 4096 they take 3.3-4.3 us per
// call against 2.0-2.8.
#ifndef RN_FWD_BF16_4096
#define RN_FWD_BF16_4096 Plan<8, 2, 4, 4>
#endif
#ifndef RN_FWD_BF16_8192
#define RN_FWD_BF16_8192 Plan<8, 2, 8, 2>
#endif
#ifndef RN_ROW_BF16_4096
#define RN_ROW_BF16_4096 Plan<8, 2, 4, 1, false>
#endif
#ifndef RN_ROW_BF16_8192
#define RN_ROW_BF16_8192 Plan<8, 2, 8, 1, false>
#endif
#ifndef RN_FWD_BF16_16384
#define RN_FWD_BF16_16384 Plan<8, 2, 16, 1>
#endif
#ifndef RN_FWD_BF16_32768
#define RN_FWD_BF16_32768 Plan<8, 4, 16, 1>
#endif
// One 8-wave workgroup per CU: with two, the waves that a CU's arbitration
// serves last leave a long tail of a few rows in flight.
#ifndef RN_BWD_BF16_1024
#define RN_BWD_BF16_1024 Plan<8, 2, 1, 8, true, 1>
#endif
#ifndef RN_BWD_BF16_2048
#define RN_BWD_BF16_2048 Plan<8, 2, 2, 4, true, 1>
#endif
#ifndef RN_BWD_BF16_4096
#define RN_BWD_BF16_4096 Plan<8, 2, 4, 2, true, 1>
#endif
#ifndef RN_BWD_BF16_8192
#define RN_BWD_BF16_8192 Plan<8, 2, 8, 1, true, 1>
#endif
#ifndef RN_BWD_BF16_16384
#define RN_BWD_BF16_16384 Plan<8, 2, 16, 1>
#endif

// ------------------------------------------------------------- forward --
using FwdPlans2B = PlanList<SegPlan<8, 8, 4, 2>,          //    64
                            SegPlan<8, 16, 4, 2>,         //   128
                            SegPlan<8, 32, 4, 2>,         //   256
                            RN_FWD_BF16_512,              //   512
                            RN_FWD_BF16_1024,             //  1024
                            RN_FWD_BF16_2048,             //  2048
                            RN_FWD_BF16_4096,             //  4096
                            RN_FWD_BF16_8192,             //  8192
                            RN_FWD_BF16_16384,            // 16384
                            RN_FWD_BF16_32768>;           // 32768
using RowPlans2B = PlanList<SegPlan<8, 8, 4, 2>, SegPlan<8, 16, 4, 2>, SegPlan<8, 32, 4, 2>,
                              RN_FWD_BF16_512, RN_FWD_BF16_1024, RN_FWD_BF16_2048,
                              RN_ROW_BF16_4096, RN_ROW_BF16_8192, RN_FWD_BF16_16384,
                              RN_FWD_BF16_32768>;
// float32 parameters take twice the registers: no 32768 plan (those rows
// take the long-row kernels).
using FwdPlans2BW = PlanList<SegPlan<8, 8, 4, 2>, SegPlan<8, 16, 4, 2>, SegPlan<8, 32, 4, 2>,
                             RN_FWD_BF16_512, RN_FWD_BF16_1024, RN_FWD_BF16_2048,
                             RN_FWD_BF16_4096, RN_FWD_BF16_8192, RN_FWD_BF16_16384>;
using RowPlans2BW = PlanList<SegPlan<8, 8, 4, 2>, SegPlan<8, 16, 4, 2>, SegPlan<8, 32, 4, 2>,
                               RN_FWD_BF16_512, RN_FWD_BF16_1024, RN_FWD_BF16_2048,
                               RN_ROW_BF16_4096, RN_ROW_BF16_8192, RN_FWD_BF16_16384>;
using FwdPlansF32 = PlanList<SegPlan<4, 8, 4, 2>,         //    32
                             SegPlan<4, 16, 4, 2>,        //    64
                             SegPlan<4, 32, 4, 2>,        //   128
                             SegPlan<4, 64, 4, 2, 1>,     //   256
                             SegPlan<4, 64, 4, 2, 2>,     //   512
                             SegPlan<4, 64, 4, 1, 4>,     //  1024
                             Plan<4, 4, 2, 2, false>,      //  2048
                             Plan<4, 4, 4, 1, false>,      //  4096
                             Plan<4, 4, 8, 1, false>,      //  8192
                             Plan<4, 4, 16, 1>>;           // 16384
using FwdPlansScalar = PlanList<SegPlan<1, 8, 4, 2>,   //     8
                                SegPlan<1, 16, 4, 2>,  //    16
                                SegPlan<1, 32, 4, 2>,  //    32
                                Plan<1, 1, 1, 4>,   //    64
                                Plan<1, 4, 1, 4>,   //   256
                                Plan<1, 4, 4, 1>,   //  1024
                                Plan<1, 4, 16, 1>,  //  4096
                                Plan<1, 8, 16, 1>>; //  8192

// ------------------------------------------------------------ backward --
#ifndef RN_BWD_BF16_128
#define RN_BWD_BF16_128 SegPlan<8, 16, 4, 1>
#endif
using BwdPlans2B = PlanList<SegPlan<8, 8, 4, 1>,    //    64
                              RN_BWD_BF16_128,      //   128
                            SegPlan<8, 32, 4, 1>,   //   256
                            Plan<8, 1, 1, 8>,       //   512
                              RN_BWD_BF16_1024,     //  1024
                              RN_BWD_BF16_2048,     //  2048
                              RN_BWD_BF16_4096,     //  4096
                              RN_BWD_BF16_8192,     //  8192
                              RN_BWD_BF16_16384>;   // 16384
// float32 rows of 16 elements per lane are too wide to double-buffer.
using BwdPlansF32 = PlanList<SegPlan<4, 8, 4, 1>,          //    32
                             SegPlan<4, 16, 4, 1>,         //    64
                             SegPlan<4, 32, 4, 1>,         //   128
                             Plan<4, 1, 1, 8>,             //   256
                             Plan<4, 2, 1, 8>,             //   512
                             Plan<4, 4, 1, 8, false>,      //  1024
                             Plan<4, 4, 2, 4, false>,      //  2048
                             Plan<4, 4, 4, 2, false>,      //  4096
                             Plan<4, 4, 8, 1, false>,      //  8192
                             Plan<4, 4, 16, 1, false>>;    // 16384
using BwdPlansScalar = PlanList<SegPlan<1, 8, 4, 1>,   //     8
                                SegPlan<1, 16, 4, 1>,  //    16
                                SegPlan<1, 32, 4, 1>,  //    32
                                Plan<1, 1, 1, 8>,   //    64
                                Plan<1, 4, 1, 8>,   //   256
                                Plan<1, 4, 4, 2>,   //  1024
                                Plan<1, 4, 16, 1>,  //  4096
                                Plan<1, 8, 16, 1>>; //  8192

// Rows past the register plans (is_long_row) walk their row in segments:
// 16-byte chunks on the vector path, single elements otherwise.
template <class... Ps>
constexpr int max_span(PlanList<Ps...>) {
    int m = 0;
    ((m = Ps::SPAN > m ? Ps::SPAN : m), ...);
    return m;
}

// VecPlans: the 16-byte path's plans; RowPlans: the same row lengths with
// one workgroup per row group wherever VecPlans run persistent teams, for
// the fused op and for inputs of fewer than 4 rows per CU.
template <class T, class W, class VecPlans, class RowPlans = VecPlans>
hipError_t launch_fwd_t(int op, const FwdArgs &a, bool vec, int cus,
                        hipStream_t s) {
    static_assert(max_span(VecPlans{}) == max_span(RowPlans{}), "one long-row limit");
    if (a.H > (vec ? max_span(VecPlans{}) : kMaxHiddenRegScalar))
        return vec ? launch_fwd_long<T, W, Vec16<T>::N>(op, a, s)
                   : launch_fwd_long<T, W, 1>(op, a, s);
    auto f = [&]<class P>() { return launch_fwd_any<T, W, P>(op, a, cus, s); };
    if (!vec) return pick_plan(FwdPlansScalar{}, a.H, f);
    const bool few = a.N < 4 * (int64_t)cus;
    return (op == OP_FUSED || few) ? pick_plan(RowPlans{}, a.H, f)
                                   : pick_plan(VecPlans{}, a.H, f);
}

template <class T, class W, class VecPlans>
int bwd_partials_t(int64_t N, int H, bool vec, int cus) {
    if (is_long_row(H, vec)) return bwd_long_partials(N, cus);
    auto f = [&]<class P>() { return bwd_grid_any<T, W, P>(N, H, cus); };
    return vec ? pick_plan_int(VecPlans{}, H, f)
               : pick_plan_int(BwdPlansScalar{}, H, f);
}

template <class T, class W, class VecPlans>
hipError_t launch_bwd_t(bool ln, bool fused, const BwdArgs &a, bool vec, int P,
                        bool colsum, int cus, void *dg, void *db, hipStream_t s) {
    if (is_long_row(a.H, vec))
        return vec ? launch_bwd_long<T, W, Vec16<T>::N>(ln, fused, a, P, colsum, dg, db, s)
                   : launch_bwd_long<T, W, 1>(ln, fused, a, P, colsum, dg, db, s);
    auto f = [&]<class Pl>() {
        return launch_bwd_any<T, W, Pl>(ln, fused, a, P, colsum, cus, dg, db, s);
    };
    return vec ? pick_plan(VecPlans{}, a.H, f)
               : pick_plan(BwdPlansScalar{}, a.H, f);
}

// Body of the translation units: the three entry points for storage pair
// S = (T activations, W parameters) with the given vector plan lists.
#define RN_DEFINE_FWD(S, T, W, ...)                                                \
    hipError_t launch_fwd_##S(int op, const FwdArgs &a, bool vec, int cus,         \
                              hipStream_t s) {                                     \
        return launch_fwd_t<T, W, __VA_ARGS__>(op, a, vec, cus, s);                \
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
