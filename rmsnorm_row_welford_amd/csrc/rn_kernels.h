// Row-normalization kernels for gfx950.
//
// Work decomposition.  A "team" of TW wavefronts (64*TW lanes) owns one row
// at a time; a workgroup holds RT teams.  Lane l of a team owns CPL chunks of
// VEC consecutive elements: chunk c covers elements [(c*64*TW + l)*VEC, +VEC),
// so each chunk step of a wave is one fully coalesced 64 x 16-byte access.
// The whole row stays in registers between the statistics and the output
// pass, so every element is read from HBM once.  Rows are addressed through
// buffer resources sized to the row: chunks at or past H load as 0 from the
// hardware range check, contribute nothing, and their stores are dropped.
//
// Workgroups are persistent: the grid is capped near the number of resident
// workgroups and each team strides over rows (grp = blockIdx.x, += gridDim.x;
// row = grp*RT + team).  gamma/beta are loaded once per team into registers,
// and each team requests its next row before it works on the current one.
//
// Statistics (fp32 throughout):
//  * LayerNorm works on x - pivot (pivot = the row's first element), so
//    sums and deviations carry the row's spread rather than its mean.
//  * TW == 1: two-pass over the register-resident row, each pass a wave64
//    sum by DPP (mean first, then the centered sum of squares).
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
// end the RT teams of a workgroup are added column-wise through LDS in team
// order and the workgroup writes ONE float32 partial row (two for
// LayerNorm).  The grid
// of kernel 1 is a small multiple of the CU count, so the partial buffer
// does not grow with N.  Kernel 2 sums the partial rows column-wise in a
// fixed order and rounds to the parameter type.  When the rows are so few
// that the partial rows would cost more than reading x and dy again, kernel
// 1 writes dx only and then forms dgamma/dbeta itself, column tile by
// column tile (the column-sum strategy, one launch).
#pragma once

#include <atomic>

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
    template <class T>
    __device__ __forceinline__ int boff(int c) const { return off(c) * (int)sizeof(T); }

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

// Row I/O through a buffer resource covering exactly the row's H elements:
// chunks past the row load as 0 and are not stored.
template <class T>
__device__ __forceinline__ rsrc_t row_rsrc(const T *row, int H) {
    return make_rsrc(row, (uint32_t)H * (uint32_t)sizeof(T));
}

template <int AUX, class T, int VEC, int CPL, int TW>
__device__ __forceinline__ void load_raw_row(rsrc_t r, const Layout<VEC, CPL, TW> &L,
                                             RawChunk<T, VEC> *v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c].template bload<AUX>(r, L.template boff<T>(c));
}

template <class T, int VEC, int CPL, int TW>
__device__ __forceinline__ void store_row(rsrc_t r, const Layout<VEC, CPL, TW> &L,
                                          const float *v) {
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        bstore_chunk<VEC>((T *)nullptr, r, L.template boff<T>(c), v + c * VEC);
}

// ----------------------------------------------------------------- forward --
// Workgroups ask for 8 waves per SIMD (<= 64 VGPRs) where that costs no
// spills: 1024-thread forward workgroups, so that two rows' workgroups
// share a CU, and single-wave rows of up to 16 two-byte elements per lane
// (LayerNorm there would otherwise take 70 registers and 7 waves).
#ifndef RN_FWD_MINW8
#define RN_FWD_MINW8 1
#endif
// Rows a prefetching (PF) forward team requests ahead of the one it works
// on: three for 2-byte activations (a 16384-element row is 8 registers per
// lane packed, so three in flight fit beside the one being reduced), one
// for float32 (the fused op's two inputs would spill).  These plans run one
// workgroup per CU, so the rows in flight per CU are what keeps HBM busy.
#ifndef RN_FWD_PF_DEPTH
#define RN_FWD_PF_DEPTH 3
#endif
// Prefetching teams walk their ring with every load and store issued (rows
// past N into empty ranges), so that the compiler's waits at the loop head
// count exactly the operations issued after each one (see fwd_kernel).
#ifndef RN_FWD_RING
#define RN_FWD_RING 1
#endif

template <class T, class W, int VEC, int CPL, int TW, int RT, int OP, bool PF>
constexpr int fwd_min_waves() {
    return ((TW * RT == 16 && !PF) ||
            (RN_FWD_MINW8 && sizeof(T) == 2 && TW == 1 && VEC * CPL <= 16))
               ? 8
               : 1;
}

// FULL: H equals the plan's span, so every chunk is inside the row and
// LayerNorm needs no masking selects.
template <class T, class W, int VEC, int CPL, int TW, int RT, int OP, bool PF,
          bool FULL = false>
__global__ __launch_bounds__(64 * TW * RT, (fwd_min_waves<T, W, VEC, CPL, TW, RT, OP, PF>()))
void fwd_kernel(const FwdArgs a) {
    using Lay = Layout<VEC, CPL, TW>;
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    constexpr int E = Lay::E;
    // values each wave posts for the cross-wave step: LayerNorm (pivot,
    // shifted mean, M2), RMSNorm the sum of squares
    constexpr int NV = (OP == OP_LN) ? 3 : 1;
    constexpr int NIN = (OP == OP_FUSED) ? 2 : 1;   // row inputs: x [, residual]
    __shared__ float red[(TW > 1) ? 2 * RT * TW * NV : 1];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int team = wave / TW;
    const int wit = wave - team * TW;
    const int H = a.H;
    const Lay L(wit * 64 + lane, H);

    RawW g[CPL];
    load_raw_row<0>(row_rsrc((const W *)a.gamma, H), L, g);
    RawW bt[(OP == OP_LN) ? CPL : 1];
    if constexpr (OP == OP_LN) {
        if (a.beta != nullptr) load_raw_row<0>(row_rsrc((const W *)a.beta, H), L, bt);
        else
#pragma unroll
            for (int c = 0; c < CPL; ++c) bt[c].zero();
    }

    // Cross-wave LayerNorm statistics: wave w shifts its n_w elements by its
    // own first element p_w and holds the two-pass mean m_w and M2_w of the
    // shifted values.  Lane w of every wave later picks up wave w's state;
    // the means are restated against wave 0's pivot, d_w = (p_w - p_0) + m_w,
    // and the states are combined with the parallel Welford merge in its
    // multi-way form: mean - p_0 = sum(n_w d_w)/H,
    // M2 = sum(M2_w + n_w (d_w - (mean - p_0))^2).  n_w depends only on H.
    float inv_cnt = 0.0f, n_lane = 0.0f;
    if constexpr (OP == OP_LN && TW > 1) {
        const float nw = (float)Lay::wave_count(wit, H);
        inv_cnt = nw > 0.0f ? 1.0f / nw : 0.0f;
        n_lane = lane < TW ? (float)Lay::wave_count(lane, H) : 0.0f;
    }

    const T *xb = (const T *)a.x;
    const T *rb = (const T *)a.res;
    const int64_t N = a.N;
    const int64_t step = (int64_t)gridDim.x * RT;

    // Software pipeline (PF): the raw chunks of the team's next rows are
    // requested before the current row is reduced and written, so HBM reads
    // stay in flight across the reductions.  Without PF each row is fetched when its turn
    // comes and latency is hidden by occupancy alone.
    // PD rows are requested ahead: a ring of PD + 1 row buffers, which the
    // loop below walks unrolled so that each buffer keeps its registers (no
    // copies from one buffer to the next).
    constexpr int PD = !PF ? 0 : (sizeof(T) == 2 && VEC * CPL <= 16) ? RN_FWD_PF_DEPTH : 1;
    constexpr int NR = PD + 1;
    Raw ring[NR][NIN][CPL];
    // URING: the ring's loads and stores are all issued, with no branch
    // around them; a row past N is read from and written to an empty range
    // (loads return 0, stores are dropped).  Branches around memory
    // operations make the compiler's wait-count analysis merge paths with
    // different outstanding operations, and at the loop head it then waits
    // for every load and store in flight, the prefetched rows included.
    constexpr bool URING = RN_FWD_RING && PD > 0;
    auto fetch = [&](int64_t row, auto &dst) {
        if constexpr (URING) {
            const bool in = row < N;
            const int64_t r = in ? row : 0;
            const uint32_t nb = in ? (uint32_t)H * (uint32_t)sizeof(T) : 0u;
            load_raw_row<RN_LOAD_AUX>(make_rsrc(xb + r * a.ldx, nb), L, dst[0]);
            if constexpr (OP == OP_FUSED)
                load_raw_row<RN_LOAD_AUX>(make_rsrc(rb + r * a.ldr, nb), L, dst[1]);
        } else if (row < N) {
            load_raw_row<RN_LOAD_AUX>(row_rsrc(xb + row * a.ldx, H), L, dst[0]);
            if constexpr (OP == OP_FUSED)
                load_raw_row<RN_LOAD_AUX>(row_rsrc(rb + row * a.ldr, H), L, dst[1]);
        } else {
#pragma unroll
            for (int i = 0; i < NIN; ++i)
#pragma unroll
                for (int c = 0; c < CPL; ++c) dst[i][c].zero();
        }
    };
    int parity = 0;
    // One row of the team: statistics, y (and h), saved statistics.
    auto process = [&](auto &cur, const int64_t row, const bool active) {
        // URING: an inactive row's stores go to empty ranges
        const uint32_t ob = active ? (uint32_t)H * (uint32_t)sizeof(T) : 0u;
        const int64_t rr = active ? row : 0;
        float v[E];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                v[c * VEC + k] = cur[0][c].get(k);
                if constexpr (OP == OP_FUSED) v[c * VEC + k] += cur[1][c].get(k);
            }
        // h is written back in the same pass, before y; every element of
        // this lane was loaded before, so h may alias x or the residual.
        if constexpr (OP == OP_FUSED) {
            if constexpr (URING) store_row<T>(make_rsrc((T *)a.h + rr * a.ldh, ob), L, v);
            else if (active) store_row<T>(row_rsrc((T *)a.h + row * a.ldh, H), L, v);
        }

        float mean = 0.0f, var;
        // rows of more than 16 elements per lane: LayerNorm's shifted values
        // are widened again from the packed chunks where used instead of
        // kept as float32 (the registers of the ring and the parameters)
        constexpr bool REW = OP == OP_LN && E > 16;
        float pv = 0.0f, mv = 0.0f;   // REW: x - mean = (x - pv) - mv
        if constexpr (OP == OP_LN) {
            // Shift by a pivot (the first element of the row, or of the
            // wave's part of it) so that the sums and deviations are formed
            // from values of the row's spread, not of its mean: with
            // |mean| >> std the float32 rounding of the mean itself would
            // otherwise dominate x - mean.  v becomes x - pivot on valid
            // elements and 0 on masked ones.
            const float pivot = lane_value(v[0], 0);
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    float &u = v[c * VEC + k];
                    u = (FULL || L.valid(c)) ? u - pivot : 0.0f;
                    s += u;
                }
            float ms;   // subtracted from the shifted values: they become x - mean
            if constexpr (TW == 1) {
                ms = wave_sum(s) * a.inv_H;
                float q = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const float d = (FULL || L.valid(c)) ? v[c * VEC + k] - ms : 0.0f;
                        q = __builtin_fmaf(d, d, q);
                    }
                var = wave_sum(q) * a.inv_H;
                mean = pivot + ms;
            } else {
                const float mw = wave_sum(s) * inv_cnt;
                if constexpr (REW) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) opaque(cur[0][c].v);
                }
                float q = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        const float u = REW ? cur[0][c].get(k) - pivot : v[c * VEC + k];
                        const float d = (FULL || L.valid(c)) ? u - mw : 0.0f;
                        q = __builtin_fmaf(d, d, q);
                    }
                q = wave_sum(q);
                float *slot = red + ((parity * RT + team) * TW) * NV;
                if (lane == 0) {
                    slot[NV * wit] = pivot;
                    slot[NV * wit + 1] = mw;
                    slot[NV * wit + 2] = q;
                }
                __syncthreads();
                const float p0 = slot[0];   // wave 0's pivot: the row's first element
                const float dl = lane < TW ? (slot[NV * lane] - p0) + slot[NV * lane + 1] : 0.0f;
                const float ql = lane < TW ? slot[NV * lane + 2] : 0.0f;
                const float m0 = wave_sum(n_lane * dl) * a.inv_H;   // mean - p0
                const float dm = dl - m0;
                var = wave_sum(__builtin_fmaf(n_lane * dm, dm, ql)) * a.inv_H;
                // this wave's shifted values minus ms are x - mean
                ms = m0 - (pivot - p0);
                mean = p0 + m0;
                parity ^= 1;
            }
            // Teams that run one workgroup per CU with deep prefetch keep the
            // float32 row (x - pivot) across the statistics.  Otherwise it is
            // widened again from the packed chunks (made opaque so the
            // compiler cannot keep the first widening live), which frees E
            // registers for occupancy.  Same operations, same bits.
            if constexpr (REW) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) opaque(cur[0][c].v);
                pv = pivot;
                mv = ms;
            } else if constexpr (PD >= 2) {
#pragma unroll
                for (int e = 0; e < E; ++e) v[e] -= ms;   // x - mean
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) opaque(cur[0][c].v);
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int k = 0; k < VEC; ++k)
                        v[c * VEC + k] = (cur[0][c].get(k) - pivot) - ms;   // x - mean
            }
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
        const float rstd = rsqrt_pos(var + a.eps);

        if (URING || active) {
            if constexpr (REW) {
                // widen the parameters per row too (not hoisted out of the loop)
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    opaque(g[c].v);
                    opaque(bt[c].v);
                }
            }
            float out[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float ge = g[e / VEC].get(e % VEC);
                if constexpr (REW) {
                    const float d = (FULL || L.valid(e / VEC))
                                        ? (cur[0][e / VEC].get(e % VEC) - pv) - mv
                                        : 0.0f;
                    out[e] = __builtin_fmaf(d * rstd, ge, bt[e / VEC].get(e % VEC));
                } else if constexpr (OP == OP_LN)
                    out[e] = __builtin_fmaf(v[e] * rstd, ge, bt[e / VEC].get(e % VEC));
                else
                    out[e] = (v[e] * rstd) * ge;
            }
            if constexpr (URING) {
                store_row<T>(make_rsrc((T *)a.y + rr * a.ldy, ob), L, out);
                // the row's statistics: lane 0 of wave 0 stores them, every
                // other lane falls past a 4-byte range (no branch)
                const int so = (wit == 0 && lane == 0) ? 0 : 4;
                if constexpr (OP == OP_LN)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(mean),
                        make_rsrc(a.mean ? a.mean + rr : a.rstd, (active && a.mean) ? 4u : 0u),
                        so, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(rstd),
                    make_rsrc(a.rstd ? a.rstd + rr : a.mean, (active && a.rstd) ? 4u : 0u), so,
                    0, 0);
            } else {
                store_row<T>(row_rsrc((T *)a.y + row * a.ldy, H), L, out);
                if (wit == 0 && lane == 0) {
                    if constexpr (OP == OP_LN) {
                        if (a.mean) a.mean[row] = mean;
                    }
                    if (a.rstd) a.rstd[row] = rstd;
                }
            }
        }
    };

    // Persistent loop over the team's rows, unrolled over the ring: the row
    // in buffer u is worked on while buffer (u + PD) % NR receives the row
    // PD steps ahead.
    int64_t grp = blockIdx.x;
    if constexpr (URING) {
        // The workgroup's K row groups: whole turns of the ring in a loop
        // with no exit inside, then the remaining K mod NR groups.  Each
        // prefetch before the loop is followed by a row's stores into an
        // empty range (nothing is written), so the loop is entered with the
        // same sequence of outstanding memory operations as it repeats with.
        const int64_t ngrp = (N + RT - 1) / RT;
        const int64_t K = ngrp > (int64_t)blockIdx.x
                              ? (ngrp - (int64_t)blockIdx.x + gridDim.x - 1) / gridDim.x
                              : 0;
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            fetch(grp * RT + team + d * step, ring[d]);
            float z[E] = {};
            const rsrc_t none = make_rsrc(a.y, 0u);
            if constexpr (OP == OP_FUSED) store_row<T>(none, L, z);
            store_row<T>(none, L, z);
            if constexpr (OP == OP_LN) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, 0);
        }
        auto slot = [&](const int u) {
            const int64_t row = grp * RT + team;
            fetch(row + PD * step, ring[(u + PD) % NR]);
            process(ring[u], row, row < N);
            grp += gridDim.x;
        };
        for (int64_t k = K / NR; k > 0; --k) {
#pragma unroll
            for (int u = 0; u < NR; ++u) slot(u);
        }
        const int rem = (int)(K % NR);
#pragma unroll
        for (int u = 0; u + 1 < NR; ++u)
            if (u < rem) slot(u);
    } else {
#pragma unroll
        for (int d = 0; d < PD; ++d) fetch(grp * RT + team + d * step, ring[d]);
        bool done = grp * RT >= N;
        while (!done) {
#pragma unroll
            for (int u = 0; u < NR; ++u) {
                if (!done) {
                    const int64_t row = grp * RT + team;
                    const bool active = row < N;
                    if (TW == 1 && !active) {
                        done = true;   // wave-uniform; single-wave teams use no barrier
                    } else {
                        if constexpr (PD > 0)
                            fetch(row + PD * step, ring[(u + PD) % NR]);
                        else
                            fetch(row, ring[u]);
                        process(ring[u], row, active);
                        grp += gridDim.x;
                        done = grp * RT >= N;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------- partial-row layout --
// Rows of up to RN_PART_COLMAJOR_MAX_H elements store the P float32 partial
// rows of a parameter column-major: the P values of column j are
// contiguous, at part[j * Pp + slot] (Pp = partial_stride(P)), so kernel 2
// reads a column with a few 16-byte loads and one wavefront reduces it.
// Workgroup b writes slot slot_of(b): the workgroups that share an XCD
// (b mod 8, as the dispatcher deals them out) take adjacent slots, so each
// column's cache line is filled from one L2; slots no workgroup owns are
// skipped.  Longer rows keep the partial rows row-major (part[slot * H + j],
// slot = b): a workgroup's partial row then leaves in whole lines, while in
// the column-major layout the 32 workgroups of an XCD each write 4 bytes of
// every line.  Measured: at 2048 row-major partials took 1.8 us off the
// LayerNorm backward; at 1024 kernel 1 gains 0.5-0.75 us and kernel 2 loses
// 0.4; at 16384 column-major stores touch more lines than an L2 can merge.
// The dbeta partials follow at part + Pp * H.
#ifndef RN_PART_COLMAJOR_MAX_H
#define RN_PART_COLMAJOR_MAX_H 512
#endif
__host__ __device__ inline bool partial_colmajor(int H) {
    return H <= RN_PART_COLMAJOR_MAX_H;
}
__device__ __forceinline__ int slot_of(int b, int P) {
    return (b & 7) * (partial_stride(P) >> 3) + (b >> 3);
}
// Does column-major slot s hold a workgroup's partial row?
__device__ __forceinline__ bool slot_used(int s, int P) {
    const int per = partial_stride(P) >> 3;
    const int x = s / per, j = s - x * per;
    return j < ((P - x + 7) >> 3);
}
// Where workgroup `b` of `P` writes column `col` of its partial row.
__device__ __forceinline__ int64_t partial_index(int b, int P, int H, int col) {
    return partial_colmajor(H) ? (int64_t)col * partial_stride(P) + slot_of(b, P)
                               : (int64_t)b * H + col;
}

// ---------------------------------------------------------------- backward --
// Rows a prefetching (PF) backward team requests ahead of the one it works
// on.
#ifndef RN_BWD_PF_DEPTH
#define RN_BWD_PF_DEPTH 1
#endif
#ifndef RN_BWD_RING
#define RN_BWD_RING 1
#endif
// LayerNorm backward: dx with the row constants folded (two instructions
// per element instead of three).
#ifndef RN_BWD_FOLD
#define RN_BWD_FOLD 1
#endif
// 1: the register plans' dx kernel takes the column tiles after its rows;
// 0: they run as a second kernel.
#ifndef RN_COLSUM_FUSED
#define RN_COLSUM_FUSED 1
#endif
// Minimum waves per SIMD asked of the dx-only kernel (column-sum strategy)
// of 16-wave teams: 8 keeps two workgroups per CU (64 registers, no spill
// for LayerNorm and RMSNorm of bf16 rows; the fused op's variant and fp16
// rows would spill and are left to the compiler).  Measured: 512 x 16384
// LayerNorm 19.0 -> 17.1 us.
#ifndef RN_BWD_DX_MINW
#define RN_BWD_DX_MINW 8
#endif
// Largest one-per-CU workgroup (in waves) whose teams keep float32 copies.
#ifndef RN_BWD_KEEP_MAXW
#define RN_BWD_KEEP_MAXW 8
#endif
// LayerNorm teams park both accumulators in LDS at once at the end (one
// barrier instead of three; twice the LDS).
#ifndef RN_BWD_MERGE_ONCE
#define RN_BWD_MERGE_ONCE 1
#endif
// Dynamic LDS floats of backward kernel 1 for a plan of RT teams (the
// teams' accumulators meet there at the end).
__host__ __device__ constexpr int bwd1_lds_floats(int RT, int H, bool ln) {
    return RT > 1 ? RT * H * ((ln && RN_BWD_MERGE_ONCE) ? 2 : 1) : 0;
}

// ACC: accumulate dy*x_hat (and dy) and write partial rows; without it the
// kernel writes dx and then takes its share of the column tiles that form
// dgamma/dbeta (the column-sum strategy).  ADD (RMSNorm only): the fused add+RMSNorm
// backward, where x is the stored h, a.add (if set) is added to dx and
// a.dx2 (if set) receives the same values as dx.
// KEEP (plans that run one workgroup of at most 8 waves per CU, which
// leaves each wave 256 registers): gamma is widened once for the whole
// loop and the float32 x_hat and g of a row are kept from the sums to the
// dx pass; otherwise only the packed chunks are kept and widened again.
// FINAL (a grid of one workgroup): the workgroup's sums are the column sums,
// written straight to dgamma/dbeta in the parameter type (the same bits
// kernel 2 would produce from the single partial row).
template <class T, class W, int VEC, int CPL, int TW, int RT, bool LN, bool PF, bool ACC,
          bool ADD = false, bool KEEP = false, bool FINAL = false>
__global__ __launch_bounds__(64 * TW * RT,
                             (!ACC && !ADD && !__is_same(T, f16_t) && TW * RT == 16)
                                 ? RN_BWD_DX_MINW
                                 : 1)
void bwd1_kernel(const BwdArgs a) {
    static_assert(!(LN && ADD), "the residual variant is RMSNorm's");
    using Lay = Layout<VEC, CPL, TW>;
    using Raw = RawChunk<T, VEC>;
    constexpr int E = Lay::E;
    constexpr int NV = LN ? 2 : 1;
    __shared__ float red[(TW > 1) ? 2 * RT * TW * NV : 1];
    extern __shared__ f32x4 acc_lds[];   // RT > 1: RT * H floats

    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int team = wave / TW;
    const int wit = wave - team * TW;
    const int H = a.H;
    const Lay L(wit * 64 + lane, H);

    static_assert(!KEEP || TW * RT <= RN_BWD_KEEP_MAXW, "KEEP needs the registers of few waves");
    RawChunk<W, VEC> g[CPL];
    load_raw_row<0>(row_rsrc((const W *)a.gamma, H), L, g);
    float gf[KEEP ? E : 1];
    if constexpr (KEEP) {
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) gf[c * VEC + k] = g[c].get(k);
    }
    float adg[ACC ? E : 1], adb[(ACC && LN) ? E : 1];
    if constexpr (ACC) {
#pragma unroll
        for (int e = 0; e < E; ++e) adg[e] = 0.0f;
        if constexpr (LN) {
#pragma unroll
            for (int e = 0; e < E; ++e) adb[e] = 0.0f;
        }
    }

    const T *xb = (const T *)a.x;
    const T *dyb = (const T *)a.dy;
    const int64_t N = a.N;
    const int64_t step = (int64_t)gridDim.x * RT;

    // x and dy stay in their storage form (bf16: two per register); x_hat
    // and g are formed from them once for the sums and once more for dx.
    // With PF the next row is requested before the current one is worked
    // on, in one of two loops:
    //  - the copying loop: the row lands in a second buffer that is copied
    //    into the first after the current row; rows past N are zero-filled
    //    without loads;
    //  - the ring (RING): rows are requested RN_BWD_PF_DEPTH turns ahead
    //    into buffers walked unrolled, with no copies.  Every load and store
    //    is issued whatever the row: rows past N (and an absent residual
    //    gradient) use empty ranges, which load 0 and store nothing, so the
    //    compiler's wait before each row counts exactly what was issued
    //    after that row's loads.
    // The ring pays on multi-wave teams that keep float copies (1.5 us at
    // 16384 x 2048); on single-wave teams and 16-wave teams the per-row range
    // set-up costs more than it saves (and 16-wave teams would spill).
    // RN_BWD_RING: 0 the copying loop everywhere, 1 the ring on multi-wave
    // teams that keep float copies, 2 the ring on every prefetching plan.
    constexpr bool RING = PF && (RN_BWD_RING == 2 || (RN_BWD_RING == 1 && KEEP && TW > 1));
    constexpr int PD = RING ? RN_BWD_PF_DEPTH : (PF ? 1 : 0);
    constexpr int NR = PD + 1;
    struct Buf {
        Raw x[CPL], dy[CPL], ad[ADD ? CPL : 1];
        float mu, s;
    };
    Buf ring[RING ? NR : 1];   // the copying loop uses cur and nxt instead
    Buf cur, nxt;
    const T *addb = (const T *)a.add;
    const bool has_add = ADD && addb != nullptr;
    auto fetch = [&](int64_t row, Buf &b) {
        if constexpr (!RING) {
            // the copying loop: rows past N are zero-filled without loads
            // (the statistics go through locals: stores to either member
            // from two branches would keep the buffer in scratch)
            float mu = 0.0f, sv = 0.0f;
            if (row < N) {
                load_raw_row<RN_LOAD_AUX>(row_rsrc(xb + row * a.ldx, H), L, b.x);
                load_raw_row<RN_LOAD_AUX>(row_rsrc(dyb + row * a.lddy, H), L, b.dy);
                if constexpr (ADD) {
                    if (has_add)
                        load_raw_row<RN_LOAD_AUX>(row_rsrc(addb + row * a.ldadd, H), L, b.ad);
                }
                if constexpr (LN) mu = a.mean[row];
                sv = a.rstd[row];
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    b.x[c].zero();
                    b.dy[c].zero();
                }
            }
            b.mu = mu;
            b.s = sv;
            return;
        }
        const bool in = row < N;
        const int64_t r = in ? row : 0;
        const uint32_t nb = in ? (uint32_t)H * (uint32_t)sizeof(T) : 0u;
        load_raw_row<RN_LOAD_AUX>(make_rsrc(xb + r * a.ldx, nb), L, b.x);
        load_raw_row<RN_LOAD_AUX>(make_rsrc(dyb + r * a.lddy, nb), L, b.dy);
        if constexpr (ADD)
            load_raw_row<RN_LOAD_AUX>(
                make_rsrc(has_add ? addb + r * a.ldadd : xb, has_add ? nb : 0u), L, b.ad);
        b.mu = LN ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  make_rsrc(a.mean + r, in ? 4u : 0u), 0, 0, 0))
                  : 0.0f;
        b.s = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.rstd + r, in ? 4u : 0u), 0, 0, 0));
    };

    int parity = 0;
    // One row of the team: dx, and its terms added to the accumulators.
    // Rows past N hold zeros: they add nothing and store nothing.
    auto process = [&](Buf &b, const int64_t row, const bool active) {
        const float cmu = b.mu, cs = b.s;
        float sg = 0.0f, sgx = 0.0f;
        float kx[KEEP ? E : 1], kg[KEEP ? E : 1];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int e = c * VEC + k;
                const float dyv = b.dy[c].get(k);
                const float xhat = (b.x[c].get(k) - cmu) * cs;
                const float gv = dyv * (KEEP ? gf[e] : g[c].get(k));
                if constexpr (KEEP) {
                    kx[e] = xhat;
                    kg[e] = gv;
                }
                if constexpr (ACC) {
                    adg[e] = __builtin_fmaf(dyv, xhat, adg[e]);
                    if constexpr (LN) adb[e] += dyv;
                }
                sg += gv;
                sgx = __builtin_fmaf(gv, xhat, sgx);
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
        // LayerNorm: dx = rstd*g + (x_hat*(-c2*rstd) + (-c1*rstd)), two
        // instructions per element with the per-row products formed once
        const float k2 = -c2 * cs, k1 = -c1 * cs;
        if constexpr (!KEEP) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                opaque(b.x[c].v);
                opaque(b.dy[c].v);
            }
        }
        float dx[E];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int e = c * VEC + k;
                const float xhat = KEEP ? kx[e] : (b.x[c].get(k) - cmu) * cs;
                float t = KEEP ? kg[e] : b.dy[c].get(k) * g[c].get(k);
                if constexpr (LN && RN_BWD_FOLD) {
                    dx[e] = __builtin_fmaf(t, cs, __builtin_fmaf(xhat, k2, k1));
                } else {
                    if constexpr (LN) t -= c1;
                    dx[e] = __builtin_fmaf(-xhat, c2, t) * cs;
                }
                if constexpr (ADD) {
                    if (has_add) dx[e] += b.ad[c].get(k);
                }
            }
        if constexpr (RING) {
            const int64_t r = active ? row : 0;
            const uint32_t ob = active ? (uint32_t)H * (uint32_t)sizeof(T) : 0u;
            store_row<T>(make_rsrc((T *)a.dx + r * a.lddx, ob), L, dx);
            if constexpr (ADD) {
                const bool two = a.dx2 != nullptr;
                store_row<T>(
                    make_rsrc(two ? (T *)a.dx2 + r * a.lddx2 : (T *)a.dx, two ? ob : 0u), L, dx);
            }
        } else if (active) {
            store_row<T>(row_rsrc((T *)a.dx + row * a.lddx, H), L, dx);
            if constexpr (ADD) {
                if (a.dx2 != nullptr)
                    store_row<T>(row_rsrc((T *)a.dx2 + row * a.lddx2, H), L, dx);
            }
        }
    };

    int64_t grp = blockIdx.x;
    if constexpr (RING) {
        // The workgroup's K row groups.
        const int64_t ngrp = (N + RT - 1) / RT;
        const int64_t K = ngrp > (int64_t)blockIdx.x
                              ? (ngrp - (int64_t)blockIdx.x + gridDim.x - 1) / gridDim.x
                              : 0;
        // Whole turns of the ring in a loop with no exit inside, then the
        // remaining K mod NR groups.  Each prefetch is followed by a row's
        // stores into an empty range (nothing is written), so the loop is
        // entered with the same sequence of outstanding memory operations
        // as it repeats with and the compiler's waits at its head need not
        // drain the rows in flight.
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            fetch(grp * RT + team + d * step, ring[d]);
            float z[E] = {};
            store_row<T>(make_rsrc(a.dx, 0u), L, z);
            if constexpr (ADD) store_row<T>(make_rsrc(a.dx, 0u), L, z);
        }
        auto slot = [&](const int u) {
            const int64_t row = grp * RT + team;
            fetch(row + PD * step, ring[(u + PD) % NR]);
            process(ring[u], row, row < N);
            grp += gridDim.x;
        };
        for (int64_t k = K / NR; k > 0; --k) {
#pragma unroll
            for (int u = 0; u < NR; ++u) slot(u);
        }
        const int rem = (int)(K % NR);
#pragma unroll
        for (int u = 0; u + 1 < NR; ++u)
            if (u < rem) slot(u);
    } else {
        // One buffer, or with PF two: the next row is requested before the
        // current one is worked on and then copied into its place.
        // Single-wave teams leave the loop at their first row past N.
        if constexpr (PF) fetch(grp * RT + team, cur);
        for (; grp * RT < N; grp += gridDim.x) {
            const int64_t row = grp * RT + team;
            const bool active = row < N;
            if constexpr (TW == 1) {
                if (!active) break;
            }
            if constexpr (PF) fetch(row + step, nxt);
            else fetch(row, cur);
            process(cur, row, active);
            if constexpr (PF) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    cur.x[c] = nxt.x[c];
                    cur.dy[c] = nxt.dy[c];
                    if constexpr (ADD) cur.ad[c] = nxt.ad[c];
                }
                cur.mu = nxt.mu;
                cur.s = nxt.s;
            }
        }
    }

    // One partial row per workgroup and parameter: row blockIdx.x holds the
    // dgamma partial, row gridDim.x + blockIdx.x the dbeta partial.  With
    // several teams, each team parks its accumulators in LDS and every
    // thread then adds a column over the teams in team order.
    if constexpr (!ACC) {
        // the column-sum strategy: dgamma/dbeta from x and dy, tile by tile
        if constexpr (RN_COLSUM_FUSED) colsum_tiles<T, W, VEC, LN, 64 * TW * RT>(a);
    } else if constexpr (RT == 1 && FINAL) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (!L.valid(c)) continue;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                store_one((W *)a.dgamma + L.off(c) + k, adg[c * VEC + k]);
                if constexpr (LN) store_one((W *)a.dbeta + L.off(c) + k, adb[c * VEC + k]);
            }
        }
    } else if constexpr (RT == 1) {
        float *pb = a.part + (int64_t)partial_stride(gridDim.x) * H;
        if (partial_colmajor(H)) {
            const int Pp = partial_stride(gridDim.x);
            const int slot = slot_of(blockIdx.x, gridDim.x);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if (!L.valid(c)) continue;
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const int64_t o = (int64_t)(L.off(c) + k) * Pp + slot;
                    a.part[o] = adg[c * VEC + k];
                    if constexpr (LN) pb[o] = adb[c * VEC + k];
                }
            }
        } else {
            const int64_t o = (int64_t)blockIdx.x * H;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                if (!L.valid(c)) continue;
                store_f32s<VEC>(a.part + o + L.off(c), adg + c * VEC);
                if constexpr (LN) store_f32s<VEC>(pb + o + L.off(c), adb + c * VEC);
            }
        }
    } else if constexpr (RN_BWD_MERGE_ONCE && NV == 2) {
        // LayerNorm: both accumulators parked at once (2 * RT * H floats of
        // LDS), one barrier, then both column sums
        float *accbuf = (float *)acc_lds;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            if (L.valid(c)) {
                store_f32s<VEC>(accbuf + team * H + L.off(c), adg + c * VEC);
                store_f32s<VEC>(accbuf + (RT + team) * H + L.off(c), adb + c * VEC);
            }
        __syncthreads();
        float *dst0 = a.part, *dst1 = a.part + (int64_t)partial_stride(gridDim.x) * H;
        for (int col = threadIdx.x; col < H; col += 64 * TW * RT) {
            float t0 = accbuf[col], t1 = accbuf[RT * H + col];
#pragma unroll
            for (int tm = 1; tm < RT; ++tm) {
                t0 += accbuf[tm * H + col];
                t1 += accbuf[(RT + tm) * H + col];
            }
            if constexpr (FINAL) {
                store_one((W *)a.dgamma + col, t0);
                store_one((W *)a.dbeta + col, t1);
            } else {
                const int64_t o = partial_index(blockIdx.x, gridDim.x, H, col);
                dst0[o] = t0;
                dst1[o] = t1;
            }
        }
    } else {
        float *accbuf = (float *)acc_lds;
#pragma unroll
        for (int p = 0; p < NV; ++p) {
            const float *acc = adg;
            if constexpr (LN) acc = p == 0 ? adg : adb;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                if (L.valid(c)) store_f32s<VEC>(accbuf + team * H + L.off(c), acc + c * VEC);
            __syncthreads();
            float *dst = a.part + (int64_t)p * partial_stride(gridDim.x) * H;
            for (int col = threadIdx.x; col < H; col += 64 * TW * RT) {
                float t = accbuf[col];
#pragma unroll
                for (int tm = 1; tm < RT; ++tm) t += accbuf[tm * H + col];
                if constexpr (FINAL) store_one((W *)(p == 0 ? a.dgamma : a.dbeta) + col, t);
                else dst[partial_index(blockIdx.x, gridDim.x, H, col)] = t;
            }
            if (p + 1 < NV) __syncthreads();
        }
    }
}

// Kernel 2: column sums of the partial rows, in a fixed order, rounded to
// the parameter type.  blockIdx.y picks dgamma (0) or dbeta (1).
//
// Column-major partials: one wavefront per column (CPW consecutive columns
// per wavefront, four wavefronts per workgroup).  Lane l adds the column's
// slots [4l, 4l+4), [4l+256, ...), ... in increasing order (slots no
// workgroup owns count as 0), then the lanes are added by the fixed wave64
// tree.
template <class T, int CPW>
__global__ __launch_bounds__(256) void bwd2_cols_kernel(const float *part, int P, int H,
                                                       T *dgamma, T *dbeta) {
    const int Pp = partial_stride(P);
    const int lane = threadIdx.x & 63;
    const int col0 = (blockIdx.x * 4 + wave_id_uniform()) * CPW;
    const float *base = part + (int64_t)blockIdx.y * Pp * H;
    T *dst = blockIdx.y == 0 ? dgamma : dbeta;
    // the loads of CPW columns and of U steps along them are issued before
    // any is summed (one step at a time would wait a memory round trip per
    // step); the sums still take each column's slots in increasing order
    constexpr int U = 8;
    float s[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) s[i] = 0.0f;
    for (int q0 = lane * 4; q0 < Pp; q0 += 256 * U) {
        f32x4 v[U][CPW];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int q = q0 + 256 * u;
                v[u][i] = (q < Pp && col0 + i < H)
                              ? *(const f32x4 *)(base + (int64_t)(col0 + i) * Pp + q)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + 256 * u;
#pragma unroll
            for (int i = 0; i < CPW; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (q < Pp && slot_used(q + k, P)) s[i] += v[u][i][k];
        }
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const float t = wave_sum(s[i]);
        if (lane == 0 && col0 + i < H) store_one(dst + col0 + i, t);
    }
}

// Row-major partials: a workgroup of THREADS threads owns COLS columns; its
// lanes form SLOTS = THREADS/COLS row slots, slot j adding the contiguous
// block of partial rows [j*R, (j+1)*R) (R = ceil(P / SLOTS)) in increasing
// order with up to 32 loads in flight.  The slot sums meet in LDS, and each
// column's SLOTS values are then added by one segment of SLOTS lanes with
// the fixed segment-sum tree.  Narrow rows take small tiles (16 columns per
// 256 threads) so that the few columns still spread over many CUs.
template <class T, int COLS, int THREADS = 1024>
__global__ __launch_bounds__(THREADS) void bwd2_rows_kernel(const float *part, int P,
                                                           int H, T *dgamma, T *dbeta) {
    constexpr int SLOTS = THREADS / COLS;
    static_assert(SLOTS == 8 || SLOTS == 16 || SLOTS == 32, "column tile");
    constexpr int CPW = 64 / SLOTS;   // columns folded per wave
    static_assert(COLS == (THREADS / 64) * CPW, "the waves fold the tile");
    __shared__ float red[SLOTS][COLS];
    const int cl = threadIdx.x % COLS;
    const int slot = threadIdx.x / COLS;
    const int col = blockIdx.x * COLS + cl;
    const int R = (P + SLOTS - 1) / SLOTS;
    const int p0 = slot * R;
    const int p1 = p0 + R < P ? p0 + R : P;
    float s = 0.0f;
    if (col < H) {
        const float *base = part + (int64_t)blockIdx.y * partial_stride(P) * H + col;
        for (int p = p0; p < p1; p += 32) {
            float v[32];
#pragma unroll
            for (int k = 0; k < 32; ++k)
                v[k] = (p + k < p1) ? base[(int64_t)(p + k) * H] : 0.0f;
#pragma unroll
            for (int k = 0; k < 32; ++k) s += v[k];
        }
    }
    red[slot][cl] = s;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int fc = (threadIdx.x >> 6) * CPW + lane / SLOTS;   // column folded
    const float t = seg_sum<SLOTS>(red[lane % SLOTS][fc]);
    const int gcol = blockIdx.x * COLS + fc;
    if (lane % SLOTS == 0 && gcol < H)
        store_one(blockIdx.y == 0 ? dgamma + gcol : dbeta + gcol, t);
}

// Columns per wavefront of kernel 2 on column-major partial rows.
#ifndef RN_BWD2_CPW
#define RN_BWD2_CPW 1
#endif
// Longest row whose row-major partial rows kernel 2 sums in small tiles.
#ifndef RN_BWD2_SMALL_H
#define RN_BWD2_SMALL_H 2048
#endif
template <class T>
hipError_t launch_bwd2(const float *part, int P, int H, bool ln, void *dg, void *db,
                       hipStream_t s) {
    const unsigned np = ln ? 2 : 1;
    if (partial_colmajor(H))
        hipLaunchKernelGGL((bwd2_cols_kernel<T, RN_BWD2_CPW>),
                           dim3((H + 4 * RN_BWD2_CPW - 1) / (4 * RN_BWD2_CPW), np), dim3(256),
                           0, s, part, P, H, (T *)dg, (T *)db);
    else if (H <= RN_BWD2_SMALL_H)
        hipLaunchKernelGGL((bwd2_rows_kernel<T, 16, 256>), dim3((H + 15) / 16, np), dim3(256),
                           0, s, part, P, H, (T *)dg, (T *)db);
    else
        hipLaunchKernelGGL((bwd2_rows_kernel<T, 64>), dim3((H + 63) / 64, np), dim3(1024),
                           0, s, part, P, H, (T *)dg, (T *)db);
    return hipGetLastError();
}

// Column sums straight from the rows: dgamma_j = sum_r dy_rj (x_rj - mean_r)
// rstd_r and dbeta_j = sum_r dy_rj.  Used instead of partial rows when the
// rows are so few that P partial rows would outweigh reading x and dy again
// (see bwd_use_colsum).  They use the saved statistics only, not dx, so the
// kernels that write dx take these tiles too, after their rows: the tiles
// then fill the tail of the dx work instead of following it as a second
// launch.  A workgroup of THREADS threads owns a tile of COLS = CL*VEC
// columns: CL lanes across the columns (one chunk each; 8 by default)
// times SL = THREADS/CL row slots; slot j adds rows j, j + SL, ... in
// increasing order, and the slots are then added in a fixed two-level order
// through LDS.  Narrow tiles make many tiles; wide ones give each slot more
// rows when the rows are few.
//
// Row iterations of a column tile whose loads are issued together.
#ifndef RN_COLSUM_UNROLL
#define RN_COLSUM_UNROLL 2
#endif
template <class T, int VEC, int THREADS, int CL_ = 8>
struct ColsumTile {
    static constexpr int CL = CL_, SL = THREADS / CL, COLS = CL * VEC;
    static constexpr int NG = THREADS / COLS;   // second-level groups of slots
    static constexpr int SPG = SL / NG;         // slots per group
    static_assert(NG * COLS == THREADS && SPG * NG == SL, "tile shape");
    static constexpr int LDS_FLOATS = SL * COLS + NG * COLS;
};

template <class T, class W, int VEC, bool LN, int THREADS, int CL_ = 8>
__device__ void colsum_tile(const BwdArgs &a, int tile, float *red) {
    using C = ColsumTile<T, VEC, THREADS, CL_>;
    constexpr int CL = C::CL, SL = C::SL, COLS = C::COLS, NG = C::NG, SPG = C::SPG;
    float *red2 = red + SL * COLS;
    const int lc = threadIdx.x % CL;
    const int slot = threadIdx.x / CL;
    const int c0 = tile * COLS + lc * VEC;
    const int H = a.H;
    const int64_t N = a.N;
    float ag[VEC], ab[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) ag[k] = ab[k] = 0.0f;
    if (c0 < H) {
        // pointers stepped by SL rows (no per-row products)
        const T *xp = (const T *)a.x + c0 + slot * a.ldx;
        const T *dp = (const T *)a.dy + c0 + slot * a.lddy;
        const int64_t xs = (int64_t)SL * a.ldx, ds = (int64_t)SL * a.lddy;
#pragma unroll RN_COLSUM_UNROLL
        for (int64_t r = slot; r < N; r += SL, xp += xs, dp += ds) {
            // packed until used
            RawChunk<T, VEC> cx, cd;
            cx.gload_nt(xp);
            cd.gload_nt(dp);
            const float mu = LN ? a.mean[r] : 0.0f;
            const float s = a.rstd[r];
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float dv = cd.get(k);
                ag[k] = __builtin_fmaf(dv, (cx.get(k) - mu) * s, ag[k]);
                if constexpr (LN) ab[k] += dv;
            }
        }
    }
#pragma unroll
    for (int p = 0; p < (LN ? 2 : 1); ++p) {
        const float *acc = p == 0 ? ag : ab;
#pragma unroll
        for (int k = 0; k < VEC; ++k) red[slot * COLS + lc * VEC + k] = acc[k];
        __syncthreads();
        const int cc = threadIdx.x % COLS, grp = threadIdx.x / COLS;
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < SPG; ++j) t += red[(grp * SPG + j) * COLS + cc];
        red2[grp * COLS + cc] = t;
        __syncthreads();
        if (threadIdx.x < COLS) {
            const int col = tile * COLS + threadIdx.x;
            if (col < H) {
                float u = 0.0f;
                for (int g = 0; g < NG; ++g) u += red2[g * COLS + threadIdx.x];
                store_one((p == 0 ? (W *)a.dgamma : (W *)a.dbeta) + col, u);
            }
        }
        __syncthreads();
    }
}

// Every column tile of the row, taken by the workgroups in turn.
template <class T, class W, int VEC, bool LN, int THREADS, int CL = 8>
__device__ void colsum_tiles(const BwdArgs &a) {
    using C = ColsumTile<T, VEC, THREADS, CL>;
    __shared__ float red[C::LDS_FLOATS];
    const int ntiles = (a.H + C::COLS - 1) / C::COLS;
    for (int t = blockIdx.x; t < ntiles; t += gridDim.x)
        colsum_tile<T, W, VEC, LN, THREADS, CL>(a, t, red);
}

// The column tiles as a kernel of their own (RN_COLSUM_FUSED = 0).
template <class T, class W, int VEC, bool LN>
__global__ __launch_bounds__(1024) void bwd_colsum_kernel(const BwdArgs a) {
    colsum_tiles<T, W, VEC, LN, 1024>(a);
}

// Workgroups the dx kernel with trailing column tiles needs: its row groups,
// or one per tile if there are more tiles (tiles of CL lanes across).
template <int VEC>
inline int64_t colsum_grid(int64_t row_groups, int H, int CL = 8) {
    const int64_t ntiles = (H + CL * VEC - 1) / (CL * VEC);
    const int64_t g = row_groups > ntiles ? row_groups : ntiles;
    return g < (1 << 20) ? g : (1 << 20);
}

// ------------------------------------------------------------------ plans --
// A plan is <VEC, CPL, TW, RT>; rows up to 64*TW*VEC*CPL elements.
// PER_CU > 0 caps the persistent backward grid at that many workgroups per
// CU (0: as many as are resident at once).
template <int VEC_, int CPL_, int TW_, int RT_, bool PF_ = true, int PER_CU_ = 0>
struct Plan {
    static constexpr int VEC = VEC_, CPL = CPL_, TW = TW_, RT = RT_;
    static constexpr int PER_CU = PER_CU_;
    // one workgroup of at most 8 waves per CU: room to keep float copies
    static constexpr bool KEEP = PER_CU_ == 1 && TW_ * RT_ <= RN_BWD_KEEP_MAXW;
    static constexpr bool PF = PF_;   // prefetch the next row into registers
    static constexpr int SPAN = 64 * TW_ * VEC_ * CPL_;
    static constexpr int THREADS = 64 * TW_ * RT_;
    static constexpr int SEG = 0;     // not a several-rows-per-wave plan
};

// Workgroups of kernel K (with `threads` threads and `lds` bytes of dynamic
// LDS) that can be resident on one CU at once, from the runtime's occupancy
// calculator (register, LDS and wave-slot limits); cached per kernel and
// LDS size in one atomic word.
template <auto K>
inline int resident_per_cu(int threads, int lds) {
    static std::atomic<int64_t> cache{-1};
    const int64_t c = cache.load(std::memory_order_relaxed);
    if (c >= 0 && (c >> 16) == lds) return (int)(c & 0xffff);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, K, threads, lds) != hipSuccess ||
        n < 1)
        n = 1;
    cache.store(((int64_t)lds << 16) | (n & 0xffff), std::memory_order_relaxed);
    return n;
}

// Persistent grid: `per_cu` workgroups per CU, never more than there are
// row groups (and, with RN_..._MIN_ROWS > 1, at least that many rows per
// team).
template <class P>
inline int persistent_grid(int64_t N, int cus, int per_cu, int min_rows) {
    int64_t groups = (N + P::RT - 1) / P::RT;
    groups = (groups + min_rows - 1) / min_rows;
    if (per_cu < 1) per_cu = 1;
    const int64_t cap = (int64_t)per_cu * cus;
    return (int)(groups < cap ? groups : cap);
}

// Build-time launch tuning (0 = the default rule): forward workgroups per
// CU, backward workgroups per CU, and the minimum rows each backward team
// of the multi-wave (wide-row) plans folds into its partial row.
#ifndef RN_FWD_PER_CU
#define RN_FWD_PER_CU 0
#endif
#ifndef RN_BWD_PER_CU
#define RN_BWD_PER_CU 0
#endif
#ifndef RN_BWD_MIN_ROWS_WIDE
#define RN_BWD_MIN_ROWS_WIDE 1
#endif

// Forward grid.  When at least two workgroups fit on a CU, one workgroup
// per row group (no persistence): the dispatcher refills CUs as rows
// finish, which streams better than a persistent loop.  When only one fits
// (1024-thread rows), a persistent grid of one workgroup per CU whose teams
// prefetch their next row.
template <class T, class W, class P, int OP, bool FULL>
hipError_t launch_fwd_kernel(const FwdArgs &a, int cus, hipStream_t s) {
    constexpr auto k = fwd_kernel<T, W, P::VEC, P::CPL, P::TW, P::RT, OP, P::PF, FULL>;
    const int resident = resident_per_cu<k>(P::THREADS, 0);
    const int per_cu = RN_FWD_PER_CU > 0 ? RN_FWD_PER_CU
                       : resident >= 2   ? (1 << 20)
                                         : resident;
    const int grid = persistent_grid<P>(a.N, cus, per_cu, 1);
    hipLaunchKernelGGL(k, dim3(grid), dim3(P::THREADS), 0, s, a);
    return hipGetLastError();
}

template <class T, class W, class P, int OP>
hipError_t launch_fwd_plan(const FwdArgs &a, int cus, hipStream_t s) {
    // LayerNorm rows that fill the span exactly need no masking selects
    if constexpr (OP == OP_LN)
        if (a.H == P::SPAN) return launch_fwd_kernel<T, W, P, OP, true>(a, cus, s);
    return launch_fwd_kernel<T, W, P, OP, false>(a, cus, s);
}

template <class T, class W, class P>
hipError_t launch_fwd_op(int op, const FwdArgs &a, int cus, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_fwd_plan<T, W, P, OP_LN>(a, cus, s);
    case OP_RMS: return launch_fwd_plan<T, W, P, OP_RMS>(a, cus, s);
    default: return launch_fwd_plan<T, W, P, OP_FUSED>(a, cus, s);
    }
}

// Backward: kernel 1's workgroup count, i.e. the number of partial rows P.
// The LayerNorm kernel has the larger footprint, so both norms use its
// occupancy, which keeps the workspace size independent of the norm.
template <class T, class W, class P>
inline int bwd_grid(int64_t N, int H, int cus) {
    if (N <= (int64_t)P::RT * RN_BWD_DECODE_ROWS) return N > 0 ? 1 : 0;
    const int lds = bwd1_lds_floats(P::RT, H, true) * (int)sizeof(float);
    constexpr auto k = bwd1_kernel<T, W, P::VEC, P::CPL, P::TW, P::RT, true, P::PF, true,
                                   false, P::KEEP>;
    int per_cu = RN_BWD_PER_CU > 0 ? RN_BWD_PER_CU : resident_per_cu<k>(P::THREADS, lds);
    if (P::PER_CU > 0 && per_cu > P::PER_CU) per_cu = P::PER_CU;
    return persistent_grid<P>(N, cus, per_cu, P::TW > 1 ? RN_BWD_MIN_ROWS_WIDE : 1);
}

template <class T, class W, class P, bool LN, bool ADD>
hipError_t launch_bwd_ln(const BwdArgs &a, int P_, bool colsum, int cus, void *dg,
                         void *db, hipStream_t s) {
    if (!colsum && P_ == 1) {
        // one workgroup holds every row: kernel 1 writes dgamma/dbeta itself
        const int lds = bwd1_lds_floats(P::RT, a.H, LN) * (int)sizeof(float);
        hipLaunchKernelGGL(
            (bwd1_kernel<T, W, P::VEC, P::CPL, P::TW, P::RT, LN, P::PF, true, ADD, P::KEEP,
                         true>),
            dim3(1), dim3(P::THREADS), lds, s, a);
        return hipGetLastError();
    }
    if (!colsum) {
        // partial rows: kernel 1 with the persistent grid P_, then kernel 2
        if (P_ > 0) {
            const int lds = bwd1_lds_floats(P::RT, a.H, LN) * (int)sizeof(float);
            hipLaunchKernelGGL(
                (bwd1_kernel<T, W, P::VEC, P::CPL, P::TW, P::RT, LN, P::PF, true, ADD,
                             P::KEEP>),
                dim3(P_), dim3(P::THREADS), lds, s, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return launch_bwd2<W>(a.part, P_, a.H, LN, dg, db, s);
    }
    // column sums: kernel 1 writes dx (forward-style grid) and then forms
    // dgamma/dbeta tile by tile from x and dy (a.dgamma, a.dbeta)
    constexpr auto k = bwd1_kernel<T, W, P::VEC, P::CPL, P::TW, P::RT, LN, P::PF, false, ADD>;
    const int resident = resident_per_cu<k>(P::THREADS, 0);
    const int rows = persistent_grid<P>(a.N, cus, resident >= 2 ? (1 << 20) : resident, 1);
    if constexpr (RN_COLSUM_FUSED) {
        const int64_t grid = colsum_grid<P::VEC>(rows, a.H);
        hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(P::THREADS), 0, s, a);
    } else {
        hipLaunchKernelGGL(k, dim3(rows), dim3(P::THREADS), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        constexpr int COLS = 8 * P::VEC;
        hipLaunchKernelGGL((bwd_colsum_kernel<T, W, P::VEC, LN>),
                           dim3((a.H + COLS - 1) / COLS), dim3(1024), 0, s, a);
    }
    return hipGetLastError();
}

template <class T, class W, class P>
hipError_t launch_bwd_plan(bool ln, bool fused, const BwdArgs &a, int P_, bool colsum,
                           int cus, void *dg, void *db, hipStream_t s) {
    if (ln) return launch_bwd_ln<T, W, P, true, false>(a, P_, colsum, cus, dg, db, s);
    if (fused) return launch_bwd_ln<T, W, P, false, true>(a, P_, colsum, cus, dg, db, s);
    return launch_bwd_ln<T, W, P, false, false>(a, P_, colsum, cus, dg, db, s);
}

}  // namespace rn
