// Row-normalization kernels for gfx950.
//
// Work decomposition.  A "team" of TW wavefronts (64*TW lanes) owns one row
// at a time; a workgroup holds RT teams.  Lane l of a team owns CPL chunks of
// VEC consecutive elements: chunk c covers elements [(c*64*TW + l)*VEC, +VEC),
// so each chunk step of a wave is one fully coalesced 64 x 16-byte access.
// The whole row stays in registers between the statistics and the output
// pass, so every element is read from HBM once.  Chunks at or past H are
// masked: they load as 0, contribute nothing, and are never stored.
//
// Workgroups are persistent: the grid is capped near the number of resident
// workgroups and each team strides over rows (grp = blockIdx.x, += gridDim.x;
// row = grp*RT + team).  gamma/beta are loaded once per team into registers.
//
// Statistics (fp32 throughout):
//  * LayerNorm works on x - pivot (pivot = the row's first element), so
//    sums and deviations carry the row's spread rather than its mean.
//  * TW == 1: two-pass over the register-resident row, each pass a wave64
//    sum by DPP/ds_swizzle (mean first, then the centered sum of squares).
//  * TW > 1 (LayerNorm): each wave takes the two-pass mean and M2 of its own
//    elements; the waves' (count, mean, M2) states meet in LDS (one barrier)
//    and are combined with the parallel Welford merge, lane w of each wave
//    holding wave w's state, by two more wave sums.
//  * RMSNorm: the wave sums of squares meet in LDS and are summed the same
//    way.
// The denominator is always H.  eps is added inside the square root.
//
// Backward.  Kernel 1 computes dx per row and accumulates dy*x_hat (and dy)
// for its columns in float32 registers across all rows a team visits; at the
// end the RT teams of a workgroup are merged through LDS in team order and
// the workgroup writes ONE float32 partial row (two for LayerNorm).  The grid
// of kernel 1 is a small multiple of the CU count, so the partial buffer
// does not grow with N.  Kernel 2 sums the partial rows column-wise in a
// fixed order and rounds to the parameter type.
#pragma once

#include "rn_device.h"
#include "rn_internal.h"

namespace rn {

// ---------------------------------------------------------------- helpers --
template <int VEC>
__device__ __forceinline__ void store_f32s(float *p, const float *v) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int k = 0; k < VEC; k += 4) {
            f32x4 w = {v[k], v[k + 1], v[k + 2], v[k + 3]};
            *(f32x4 *)(p + k) = w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) p[k] = v[k];
    }
}

// Lane layout of one team: chunk c of lane tl starts at element
// c*64*TW*VEC + tl*VEC and is valid when that is below H (VEC divides H, so
// a chunk is either wholly inside the row or wholly past its end).
template <int VEC, int CPL, int TW>
struct Layout {
    static constexpr int TL = 64 * TW;
    static constexpr int E = VEC * CPL;
    static constexpr int STEP = TL * VEC;   // elements between chunks
    int base;
    int H;

    __device__ __forceinline__ Layout(int tl, int H_) : base(tl * VEC), H(H_) {}
    __device__ __forceinline__ int off(int c) const { return c * STEP + base; }
    __device__ __forceinline__ bool valid(int c) const { return off(c) < H; }

    // Number of valid elements held by wave w of the team.
    __device__ static __forceinline__ int wave_count(int w, int H) {
        const int nch = H / VEC;
        int n = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            int k = nch - (c * TL + w * 64);
            n += k < 0 ? 0 : (k > 64 ? 64 : k);
        }
        return n * VEC;
    }
};

template <class T, int VEC, int CPL, int TW, bool NT>
__device__ __forceinline__ void load_row(const T *row, const Layout<VEC, CPL, TW> &L,
                                         float *v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (L.valid(c)) {
            load_chunk<VEC, NT>(row + L.off(c), v + c * VEC);
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) v[c * VEC + k] = 0.0f;
        }
    }
}

template <class T, int VEC, int CPL, int TW>
__device__ __forceinline__ void load_raw_row(const T *row, const Layout<VEC, CPL, TW> &L,
                                             RawChunk<T, VEC> *v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        if (L.valid(c)) v[c].load(row + L.off(c));
        else v[c].zero();
    }
}

template <class T, int VEC, int CPL, int TW, bool NT>
__device__ __forceinline__ void store_row(T *row, const Layout<VEC, CPL, TW> &L,
                                          const float *v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        if (L.valid(c)) store_chunk<VEC, NT>(row + L.off(c), v + c * VEC);
}

// ----------------------------------------------------------------- forward --
template <class T, int VEC, int CPL, int TW, int RT, int OP>
__global__ __launch_bounds__(64 * TW * RT) void fwd_kernel(const FwdArgs a) {
    using Lay = Layout<VEC, CPL, TW>;
    constexpr int E = Lay::E;
    constexpr int NV = (OP == OP_LN) ? 2 : 1;
    __shared__ float red[(TW > 1) ? 2 * RT * TW * NV : 1];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int team = wave / TW;
    const int wit = wave - team * TW;
    const int H = a.H;
    const Lay L(wit * 64 + lane, H);

    RawChunk<T, VEC> g[CPL];
    load_raw_row<T, VEC, CPL, TW>((const T *)a.gamma, L, g);
    RawChunk<T, VEC> bt[(OP == OP_LN) ? CPL : 1];
    if constexpr (OP == OP_LN) {
        if (a.beta != nullptr) load_raw_row<T, VEC, CPL, TW>((const T *)a.beta, L, bt);
        else
#pragma unroll
            for (int c = 0; c < CPL; ++c) bt[c].zero();
    }

    // Cross-wave LayerNorm statistics: wave w holds the two-pass mean m_w and
    // M2_w of its n_w elements.  Lane w of every wave later picks up wave w's
    // state, and the states are combined with the parallel Welford merge in
    // its multi-way form: mean = sum(n_w m_w)/H,
    // M2 = sum(M2_w + n_w (m_w - mean)^2).  n_w depends only on H.
    float inv_cnt = 0.0f, n_lane = 0.0f;
    if constexpr (OP == OP_LN && TW > 1) {
        const float nw = (float)Lay::wave_count(wit, H);
        inv_cnt = nw > 0.0f ? 1.0f / nw : 0.0f;
        n_lane = lane < TW ? (float)Lay::wave_count(lane, H) : 0.0f;
    }

    const int64_t N = a.N;
    int parity = 0;
    for (int64_t grp = blockIdx.x; grp * RT < N; grp += gridDim.x) {
        const int64_t row = grp * RT + team;
        const bool active = row < N;
        if constexpr (TW == 1) {
            if (!active) break;
        }
        float v[E];
        if constexpr (OP == OP_FUSED) {
            float r[E];
            if (active) {
                load_row<T, VEC, CPL, TW, true>((const T *)a.x + row * a.ldx, L, v);
                load_row<T, VEC, CPL, TW, true>((const T *)a.res + row * a.ldr, L, r);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = r[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] += r[e];
            // h is written back in the same pass, before y; every element of
            // this lane was loaded above, so h may alias x or the residual.
            if (active) store_row<T, VEC, CPL, TW, false>((T *)a.h + row * a.ldh, L, v);
        } else {
            if (active) {
                load_row<T, VEC, CPL, TW, true>((const T *)a.x + row * a.ldx, L, v);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] = 0.0f;
            }
        }

        float mean = 0.0f, var;
        if constexpr (OP == OP_LN) {
            // Shift by a pivot (the row's first element) so that the sums and
            // deviations are formed from values of the row's spread, not of
            // its mean: with |mean| >> std the float32 rounding of the mean
            // itself would otherwise dominate x - mean.  v becomes x - pivot
            // on valid elements and 0 on masked ones.
            float pivot;
            if constexpr (TW == 1) {
                pivot = lane_value(v[0], 0);
            } else {
                pivot = 0.0f;
                if (active) load_chunk<1, false>((const T *)a.x + row * a.ldx, &pivot);
            }
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    float &u = v[c * VEC + k];
                    u = L.valid(c) ? u - pivot : 0.0f;
                    s += u;
                }
            float ms;   // mean of the shifted row
            if constexpr (TW == 1) {
                ms = wave_sum(s) * a.inv_H;
                float q = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const float d = L.valid(c) ? v[c * VEC + k] - ms : 0.0f;
                        q = __builtin_fmaf(d, d, q);
                    }
                var = wave_sum(q) * a.inv_H;
            } else {
                const float mw = wave_sum(s) * inv_cnt;
                float q = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const float d = L.valid(c) ? v[c * VEC + k] - mw : 0.0f;
                        q = __builtin_fmaf(d, d, q);
                    }
                q = wave_sum(q);
                float *slot = red + ((parity * RT + team) * TW) * 2;
                if (lane == 0) {
                    slot[2 * wit] = mw;
                    slot[2 * wit + 1] = q;
                }
                __syncthreads();
                const float ml = lane < TW ? slot[2 * lane] : 0.0f;
                const float ql = lane < TW ? slot[2 * lane + 1] : 0.0f;
                ms = wave_sum(n_lane * ml) * a.inv_H;
                const float dm = ml - ms;
                var = wave_sum(__builtin_fmaf(n_lane * dm, dm, ql)) * a.inv_H;
                parity ^= 1;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] -= ms;   // v = x - mean
            mean = pivot + ms;
        } else {
            float q = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) q = __builtin_fmaf(v[e], v[e], q);
            q = wave_sum(q);
            if constexpr (TW > 1) {
                float *slot = red + (parity * RT + team) * TW;
                if (lane == 0) slot[wit] = q;
                __syncthreads();
                q = wave_sum(lane < TW ? slot[lane] : 0.0f);
                parity ^= 1;
            }
            var = q * a.inv_H;
        }
        const float rstd = 1.0f / __builtin_sqrtf(var + a.eps);

        if (active) {
            float out[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float ge = g[e / VEC].get(e % VEC);
                if constexpr (OP == OP_LN)
                    out[e] = __builtin_fmaf(v[e] * rstd, ge, bt[e / VEC].get(e % VEC));
                else
                    out[e] = (v[e] * rstd) * ge;
            }
            store_row<T, VEC, CPL, TW, false>((T *)a.y + row * a.ldy, L, out);
            if (wit == 0 && lane == 0) {
                if constexpr (OP == OP_LN) {
                    if (a.mean) a.mean[row] = mean;
                }
                if (a.rstd) a.rstd[row] = rstd;
            }
        }
    }
}

// ---------------------------------------------------------------- backward --
template <class T, int VEC, int CPL, int TW, int RT, bool LN>
__global__ __launch_bounds__(64 * TW * RT) void bwd1_kernel(const BwdArgs a) {
    using Lay = Layout<VEC, CPL, TW>;
    constexpr int E = Lay::E;
    constexpr int NV = LN ? 2 : 1;
    __shared__ float red[(TW > 1) ? 2 * RT * TW * NV : 1];
    extern __shared__ float accbuf[];   // RT > 1: NV * H floats

    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int team = wave / TW;
    const int wit = wave - team * TW;
    const int H = a.H;
    const Lay L(wit * 64 + lane, H);

    RawChunk<T, VEC> g[CPL];
    load_raw_row<T, VEC, CPL, TW>((const T *)a.gamma, L, g);
    float adg[E], adb[LN ? E : 1];
#pragma unroll
    for (int e = 0; e < E; ++e) adg[e] = 0.0f;
    if constexpr (LN) {
#pragma unroll
        for (int e = 0; e < E; ++e) adb[e] = 0.0f;
    }

    const int64_t N = a.N;
    int parity = 0;
    for (int64_t grp = blockIdx.x; grp * RT < N; grp += gridDim.x) {
        const int64_t row = grp * RT + team;
        const bool active = row < N;
        if constexpr (TW == 1) {
            if (!active) break;
        }
        float xh[E], gg[E];
        float mu = 0.0f, s = 0.0f;
        if (active) {
            load_row<T, VEC, CPL, TW, true>((const T *)a.x + row * a.ldx, L, xh);
            load_row<T, VEC, CPL, TW, true>((const T *)a.dy + row * a.lddy, L, gg);
            if constexpr (LN) mu = a.mean[row];
            s = a.rstd[row];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) xh[e] = gg[e] = 0.0f;
        }
        // Masked elements have dy = 0, so they add nothing below.
        float sg = 0.0f, sgx = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float dyv = gg[e];
            const float xhat = (xh[e] - mu) * s;
            const float gv = dyv * g[e / VEC].get(e % VEC);
            adg[e] = __builtin_fmaf(dyv, xhat, adg[e]);
            if constexpr (LN) adb[e] += dyv;
            sg += gv;
            sgx = __builtin_fmaf(gv, xhat, sgx);
            xh[e] = xhat;
            gg[e] = gv;
        }
        if constexpr (LN) wave_sum2(sg, sgx);
        else sgx = wave_sum(sgx);
        if constexpr (TW > 1) {
            float *slot = red + ((parity * RT + team) * TW) * NV;
            if (lane == 0) {
                slot[NV * wit] = sgx;
                if constexpr (LN) slot[NV * wit + 1] = sg;
            }
            __syncthreads();
            sgx = lane < TW ? slot[NV * lane] : 0.0f;
            if constexpr (LN) {
                sg = lane < TW ? slot[NV * lane + 1] : 0.0f;
                wave_sum2(sg, sgx);
            } else {
                sgx = wave_sum(sgx);
            }
            parity ^= 1;
        }
        const float c1 = LN ? sg * a.inv_H : 0.0f;
        const float c2 = sgx * a.inv_H;
        if (active) {
            float dx[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float t = gg[e];
                if constexpr (LN) t -= c1;
                dx[e] = __builtin_fmaf(-xh[e], c2, t) * s;
            }
            store_row<T, VEC, CPL, TW, false>((T *)a.dx + row * a.lddx, L, dx);
        }
    }

    // One partial row per workgroup (two for LayerNorm), teams merged in
    // order 0, 1, ..., RT-1.
    float *pg = a.part + (int64_t)blockIdx.x * H;
    float *pb = a.part + ((int64_t)gridDim.x + blockIdx.x) * H;
    if constexpr (RT == 1) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (!L.valid(c)) continue;
            store_f32s<VEC>(pg + L.off(c), adg + c * VEC);
            if constexpr (LN) store_f32s<VEC>(pb + L.off(c), adb + c * VEC);
        }
    } else {
        for (int t = 0; t < RT; ++t) {
            if (team == t) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    if (!L.valid(c)) continue;
                    float vg[VEC], vb[VEC];
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const int col = L.off(c) + k;
                        vg[k] = t > 0 ? accbuf[col] + adg[c * VEC + k] : adg[c * VEC + k];
                        if constexpr (LN)
                            vb[k] = t > 0 ? accbuf[H + col] + adb[c * VEC + k]
                                          : adb[c * VEC + k];
                    }
                    if (t < RT - 1) {
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            accbuf[L.off(c) + k] = vg[k];
                            if constexpr (LN) accbuf[H + L.off(c) + k] = vb[k];
                        }
                    } else {
                        store_f32s<VEC>(pg + L.off(c), vg);
                        if constexpr (LN) store_f32s<VEC>(pb + L.off(c), vb);
                    }
                }
            }
            if (t < RT - 1) __syncthreads();
        }
    }
}

// Kernel 2: column sums of the partial rows.  Block (64 columns x 16
// waves); wave w adds rows w, w+16, ... of its 64 columns in increasing
// order, then the 16 wave sums are added in wave order.  blockIdx.y picks
// dgamma (0) or dbeta (1).
template <class T>
__global__ __launch_bounds__(1024) void bwd2_kernel(const float *part, int P,
                                                   int H, T *dgamma, T *dbeta) {
    __shared__ float red[16][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;
    const float *base = part + (int64_t)blockIdx.y * P * H;
    float s = 0.0f;
    if (col < H) {
        int p = wave;
#pragma unroll 8
        for (; p < P; p += 16) s += base[(int64_t)p * H + col];
    }
    red[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && col < H) {
        float t = red[0][lane];
#pragma unroll
        for (int w = 1; w < 16; ++w) t += red[w][lane];
        store_one(blockIdx.y == 0 ? dgamma + col : dbeta + col, t);
    }
}

// ------------------------------------------------------------------ plans --
// A plan is <VEC, CPL, TW, RT>; rows up to 64*TW*VEC*CPL elements.
template <int VEC_, int CPL_, int TW_, int RT_>
struct Plan {
    static constexpr int VEC = VEC_, CPL = CPL_, TW = TW_, RT = RT_;
    static constexpr int SPAN = 64 * TW_ * VEC_ * CPL_;
    static constexpr int THREADS = 64 * TW_ * RT_;
};

// Persistent grid: enough workgroups for `waves_per_cu` resident waves per
// CU, never more than there are row groups.
template <class P>
inline int persistent_grid(int64_t N, int cus, int waves_per_cu) {
    const int64_t groups = (N + P::RT - 1) / P::RT;
    int64_t per_cu = waves_per_cu / (P::TW * P::RT);
    if (per_cu < 1) per_cu = 1;
    const int64_t cap = per_cu * cus;
    return (int)(groups < cap ? groups : cap);
}

template <class T, class P, int OP>
hipError_t launch_fwd_plan(const FwdArgs &a, int cus, hipStream_t s) {
    const int grid = persistent_grid<P>(a.N, cus, 32);
    hipLaunchKernelGGL((fwd_kernel<T, P::VEC, P::CPL, P::TW, P::RT, OP>),
                       dim3(grid), dim3(P::THREADS), 0, s, a);
    return hipGetLastError();
}

template <class T, class P>
hipError_t launch_fwd_op(int op, const FwdArgs &a, int cus, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_fwd_plan<T, P, OP_LN>(a, cus, s);
    case OP_RMS: return launch_fwd_plan<T, P, OP_RMS>(a, cus, s);
    default: return launch_fwd_plan<T, P, OP_FUSED>(a, cus, s);
    }
}

// Backward: kernel 1 partial-row count for a plan.
template <class P>
inline int bwd_grid(int64_t N, int cus) {
    // 16 resident waves per CU: two 512-thread or one 1024-thread
    // workgroup(s) per CU, i.e. P = 2*CUs or 1*CUs partial rows.
    return persistent_grid<P>(N, cus, 16);
}

template <class T, class P>
hipError_t launch_bwd_plan(bool ln, const BwdArgs &a, int P_, void *dg,
                           void *db, hipStream_t s) {
    if (P_ > 0) {
        const int lds = P::RT > 1 ? (ln ? 2 : 1) * a.H * (int)sizeof(float) : 0;
        if (ln)
            hipLaunchKernelGGL((bwd1_kernel<T, P::VEC, P::CPL, P::TW, P::RT, true>),
                               dim3(P_), dim3(P::THREADS), lds, s, a);
        else
            hipLaunchKernelGGL((bwd1_kernel<T, P::VEC, P::CPL, P::TW, P::RT, false>),
                               dim3(P_), dim3(P::THREADS), lds, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd2_kernel<T>), dim3((a.H + 63) / 64, ln ? 2 : 1),
                       dim3(1024), 0, s, a.part, P_, a.H, (T *)dg, (T *)db);
    return hipGetLastError();
}

}  // namespace rn
