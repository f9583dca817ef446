// Short rows: several rows per wavefront.
//
// For rows of at most SEG*VEC*CPL elements a wave is cut into 64/SEG
// segments of SEG lanes (SEG = 8, 16, 32 or 64); segment s owns one row and
// lane sl of it holds the CPL chunks of VEC elements starting at
// (c*SEG + sl)*VEC.  All lanes of a wave stay busy on rows far shorter than
// the wave's 64*VEC-element reach, and a wave moves 64 chunks per access
// instead of H/VEC.  With SEG = 64 this is one row per wave, as in
// fwd_kernel, but with IT rows of each wave in flight at once.
//
// Addressing.  A buffer resource must be wave-uniform, so it covers the
// wave's whole group of rows [row0, row0 + n): it starts at row row0 and ends
// at the last row's H-th element.  Lane offsets are s*ld + sl*VEC elements;
// a chunk at or past H gets an offset beyond every group's range, so it
// loads as 0 and its store is dropped, and rows of the group at or past N
// fall beyond the resource's end the same way.  The host uses these kernels
// only when (64/SEG)*ld*sizeof(T) < 2^31 for every row tensor, so offsets fit
// in 32 bits.
//
// Statistics are the row-per-wave kernels' (two-pass over register values,
// LayerNorm shifted by the row's first element), with sums over a segment
// instead of a wave.
#pragma once

#include "rn_kernels.h"

namespace rn {

// The value lane `src` holds, fetched by every lane (ds_bpermute).
__device__ __forceinline__ float lane_pull(float v, int src) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

constexpr uint32_t kOffOOB = 0x80000000u;   // beyond every group's range

// Resource over rows [row0, row0 + n) of a tensor with row stride ld; for
// n <= 0 an empty range (every access falls outside it).
template <class T>
__device__ __forceinline__ rsrc_t group_rsrc(const void *base, int64_t row0, int n,
                                             int64_t ld, int H) {
    const T *p = (const T *)base + (n > 0 ? row0 : 0) * ld;
    return make_rsrc(
        p, n > 0 ? (uint32_t)(((int64_t)(n - 1) * ld + H) * (int64_t)sizeof(T)) : 0u);
}

// Byte offset of lane (seg, sl)'s chunk, or kOffOOB when the chunk is past H.
template <class T, int VEC>
__device__ __forceinline__ uint32_t seg_off(int seg, int sl, int64_t ld, bool valid) {
    return valid ? (uint32_t)(((int64_t)seg * ld + sl * VEC) * (int64_t)sizeof(T)) : kOffOOB;
}

// Sum over a segment; a whole-wave segment uses the wave sum.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (SEG == 64) return wave_sum(v);
    else return seg_sum<SEG>(v);
}

// Forward.  Wave w of workgroup b owns IT consecutive groups of 64/SEG rows
// starting at row ((b*WPG + w)*IT)*(64/SEG); all IT groups are requested
// before the first is reduced.  One workgroup per WPG*IT groups (not
// persistent): the dispatcher keeps every CU fed.  FULL: H equals the
// plan's span, so every chunk is inside the row and LayerNorm needs no
// masking selects.
template <class T, class W, int VEC, int SEG, int CPL, int WPG, int IT, int OP,
          bool FULL = false>
__global__ __launch_bounds__(64 * WPG, (sizeof(T) == 2 && sizeof(W) == 2 && VEC * CPL <= 16) ? 8 : 1)
void fwd_seg_kernel(const FwdArgs a) {
    constexpr int RPW = 64 / SEG;
    constexpr int E = VEC * CPL;
    // The workgroup's rows are consecutive: their statistics meet in LDS and
    // go out in one coalesced store per output, not one small store per
    // segment (scattered 4-16 byte writes cost several times their size).
    constexpr int WROWS = WPG * IT * RPW;
    static_assert(WROWS <= 64, "one wave stores the workgroup's statistics");
    constexpr int NST = (OP == OP_LN) ? 2 : 1;
    __shared__ float stats[NST][WROWS];
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int seg = lane / SEG, sl = lane % SEG;
    const int H = a.H;
    const int64_t N = a.N;
    bool valid[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) valid[c] = FULL || (c * SEG + sl) * VEC < H;
    const int64_t row_base = (int64_t)blockIdx.x * WROWS;   // the workgroup's first row
    const int64_t wrow = row_base + (int64_t)wave * (IT * RPW);

    RawW g[CPL], bt[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const uint32_t poff =
            valid[c] ? (uint32_t)((c * SEG + sl) * VEC * (int)sizeof(W)) : kOffOOB;
        g[c].template bload<0>(row_rsrc((const W *)a.gamma, H), poff);
        if constexpr (OP == OP_LN) {
            if (a.beta != nullptr)
                bt[c].template bload<0>(row_rsrc((const W *)a.beta, H), poff);
            else
                bt[c].zero();
        }
    }

    // Every group's loads are issued, those of groups past N into an empty
    // range (they return 0 and touch no memory): with no branch around them
    // the compiler's wait before each group counts exactly the operations
    // issued after it, instead of draining the earlier groups' stores.
    Raw cx[IT][CPL], cr[(OP == OP_FUSED) ? IT : 1][CPL];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int64_t row0 = wrow + (int64_t)i * RPW;
        const int64_t left = N - row0;
        const int n = left <= 0 ? 0 : (left < RPW ? (int)left : RPW);
        const rsrc_t rx = group_rsrc<T>(a.x, row0, n, a.ldx, H);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            cx[i][c].template bload<RN_LOAD_AUX>(
                rx, seg_off<T, VEC>(seg, c * SEG + sl, a.ldx, valid[c]));
        if constexpr (OP == OP_FUSED) {
            const rsrc_t rr = group_rsrc<T>(a.res, row0, n, a.ldr, H);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                cr[i][c].template bload<RN_LOAD_AUX>(
                    rr, seg_off<T, VEC>(seg, c * SEG + sl, a.ldr, valid[c]));
        }
    }

#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int64_t row0 = wrow + (int64_t)i * RPW;
        if (row0 >= N) break;
        const int n = (int)(N - row0 < RPW ? N - row0 : RPW);
        float v[E];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                v[c * VEC + k] = cx[i][c].get(k);
                if constexpr (OP == OP_FUSED) v[c * VEC + k] += cr[i][c].get(k);
            }
        // h goes out before y; every element of this lane is already loaded,
        // so h may alias x or the residual.
        if constexpr (OP == OP_FUSED) {
            const rsrc_t rh = group_rsrc<T>(a.h, row0, n, a.ldh, H);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                bstore_chunk<VEC>((T *)nullptr, rh,
                                  seg_off<T, VEC>(seg, c * SEG + sl, a.ldh, valid[c]),
                                  v + c * VEC);
        }

        float mean = 0.0f, var;
        if constexpr (OP == OP_LN) {
            float pivot;   // the row's first element
            if constexpr (SEG == 64) pivot = lane_value(v[0], 0);
            else pivot = lane_pull(v[0], seg * SEG);
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    float &u = v[c * VEC + k];
                    u = valid[c] ? u - pivot : 0.0f;
                    s += u;
                }
            const float ms = segment_sum<SEG>(s) * a.inv_H;
            float q = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    float &u = v[c * VEC + k];
                    u = valid[c] ? u - ms : 0.0f;   // x - mean
                    q = __builtin_fmaf(u, u, q);
                }
            var = segment_sum<SEG>(q) * a.inv_H;
            mean = pivot + ms;
        } else {
            float q = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) q = __builtin_fmaf(v[e], v[e], q);
            var = segment_sum<SEG>(q) * a.inv_H;
        }
        const float rstd = rsqrt_pos(var + a.eps);

        float out[E];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int e = c * VEC + k;
                if constexpr (OP == OP_LN)
                    out[e] = __builtin_fmaf(v[e] * rstd, g[c].get(k), bt[c].get(k));
                else
                    out[e] = (v[e] * rstd) * g[c].get(k);
            }
        const rsrc_t ry = group_rsrc<T>(a.y, row0, n, a.ldy, H);
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            bstore_chunk<VEC>((T *)nullptr, ry,
                              seg_off<T, VEC>(seg, c * SEG + sl, a.ldy, valid[c]),
                              out + c * VEC);
        if (sl == 0) {
            const int lr = (wave * IT + i) * RPW + seg;   // row0 + seg - row_base
            if constexpr (OP == OP_LN) stats[1][lr] = mean;
            stats[0][lr] = rstd;
        }
    }
    __syncthreads();
    if (wave == 0 && lane < WROWS && row_base + lane < N) {
        if constexpr (OP == OP_LN) {
            if (a.mean) a.mean[row_base + lane] = stats[1][lane];
        }
        if (a.rstd) a.rstd[row_base + lane] = stats[0][lane];
    }
}

// The short-row backward requests a wave's next row group before it works on
// the current one (1), or fetches each group when its turn comes (0).
#ifndef RN_SEG_BWD_PF
#define RN_SEG_BWD_PF 1
#endif

// Backward kernel 1.  Persistent: wave w of workgroup b takes row groups
// b*WPG + w, += gridDim.x*WPG, each of 64/SEG rows; every lane accumulates
// dy*x_hat (and dy) for its VEC columns over all its rows.  At the end the
// WPG*(64/SEG) segments of the workgroup are added column-wise through LDS,
// in segment order, into ONE float32 partial row (two for LayerNorm), as in
// bwd1_kernel.  ADD: the fused add+RMSNorm variant (a.add added to dx, a.dx2
// a second copy).
// FINAL (a grid of one workgroup): the column sums go straight to
// dgamma/dbeta in the parameter type, as in bwd1_kernel.
template <class T, class W, int VEC, int SEG, int WPG, bool LN, bool ADD, bool FINAL = false>
__global__ __launch_bounds__(64 * WPG) void bwd1_seg_kernel(const BwdArgs a) {
    static_assert(!(LN && ADD), "the residual variant is RMSNorm's");
    constexpr int RPW = 64 / SEG;
    constexpr int SPAN = SEG * VEC;
    constexpr int SLOTS = WPG * RPW;
    using Raw = RawChunk<T, VEC>;
    __shared__ float acc[SLOTS * SPAN];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id_uniform();
    const int seg = lane / SEG, sl = lane % SEG;
    const int H = a.H;
    const int64_t N = a.N;
    const bool valid = sl * VEC < H;

    RawChunk<W, VEC> g;
    g.template bload<0>(row_rsrc((const W *)a.gamma, H),
                        valid ? (uint32_t)(sl * VEC * (int)sizeof(W)) : kOffOOB);
    float adg[VEC], adb[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) adg[k] = adb[k] = 0.0f;
    const T *addb = (const T *)a.add;
    const bool has_add = ADD && addb != nullptr;

    const int64_t gstep = (int64_t)gridDim.x * WPG;
    // A row group's chunks and statistics.  Every group issues the same
    // loads through wave-uniform buffer resources: a group past N reads an
    // empty range (0, nothing touched), and the statistics of row seg are
    // the word at seg*4 of a range of n words.
    struct Grp {
        Raw cx, cdy, cad;
        float mu, s;
    };
    auto rows_in = [&](int64_t gi) -> int {
        const int64_t left = N - gi * RPW;
        return left <= 0 ? 0 : (left < RPW ? (int)left : RPW);
    };
    auto fetch = [&](int64_t gi, Grp &b) {
        const int n = rows_in(gi);
        const int64_t r0 = n > 0 ? gi * RPW : 0;
        b.cx.template bload<RN_LOAD_AUX>(group_rsrc<T>(a.x, r0, n, a.ldx, H),
                                         seg_off<T, VEC>(seg, sl, a.ldx, valid));
        b.cdy.template bload<RN_LOAD_AUX>(group_rsrc<T>(a.dy, r0, n, a.lddy, H),
                                          seg_off<T, VEC>(seg, sl, a.lddy, valid));
        if constexpr (ADD)
            b.cad.template bload<RN_LOAD_AUX>(
                group_rsrc<T>(has_add ? addb : (const T *)a.x, r0, has_add ? n : 0,
                              has_add ? a.ldadd : a.ldx, H),
                seg_off<T, VEC>(seg, sl, has_add ? a.ldadd : a.ldx, valid));
        const uint32_t so = (uint32_t)seg * 4u;
        b.mu = LN ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               make_rsrc(a.mean + r0, 4u * n), so, 0, 0))
                  : 0.0f;
        b.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            make_rsrc(a.rstd + r0, 4u * n), so, 0, 0));
    };
    // dx of row group gi (n > 0 rows) from its fetched chunks
    auto work = [&](const Grp &b, int64_t gi) {
        const int64_t row0 = gi * RPW;
        const int n = rows_in(gi);
        const float mu = b.mu, s = b.s;
        // Masked elements and rows past N have dy = 0 and add nothing.
        float sg = 0.0f, sgx = 0.0f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float dyv = b.cdy.get(k);
            const float xhat = (b.cx.get(k) - mu) * s;
            const float gv = dyv * g.get(k);
            adg[k] = __builtin_fmaf(dyv, xhat, adg[k]);
            if constexpr (LN) adb[k] += dyv;
            sg += gv;
            sgx = __builtin_fmaf(gv, xhat, sgx);
        }
        if constexpr (LN) sg = seg_sum<SEG>(sg);
        sgx = seg_sum<SEG>(sgx);
        const float c1 = LN ? sg * a.inv_H : 0.0f;
        const float c2 = sgx * a.inv_H;
        const float k2 = -c2 * s, k1 = -c1 * s;   // as in bwd1_kernel
        float dx[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float xhat = (b.cx.get(k) - mu) * s;
            float t = b.cdy.get(k) * g.get(k);
            if constexpr (LN && RN_BWD_FOLD) {
                dx[k] = __builtin_fmaf(t, s, __builtin_fmaf(xhat, k2, k1));
            } else {
                if constexpr (LN) t -= c1;
                dx[k] = __builtin_fmaf(-xhat, c2, t) * s;
            }
            if constexpr (ADD) dx[k] += b.cad.get(k);
        }
        bstore_chunk<VEC>((T *)nullptr, group_rsrc<T>(a.dx, row0, n, a.lddx, H),
                          seg_off<T, VEC>(seg, sl, a.lddx, valid), dx);
        if constexpr (ADD) {
            // no second copy: the same store into an empty range
            const bool two = a.dx2 != nullptr;
            bstore_chunk<VEC>((T *)nullptr,
                              group_rsrc<T>(two ? a.dx2 : a.dx, row0, two ? n : 0,
                                            two ? a.lddx2 : a.lddx, H),
                              seg_off<T, VEC>(seg, sl, two ? a.lddx2 : a.lddx, valid), dx);
        }
    };
    int64_t gi = (int64_t)blockIdx.x * WPG + wave;
    if constexpr (RN_SEG_BWD_PF) {
        // Two buffers in turn: a wave's next group is requested before it
        // works on the current one (a copy between the buffers would make
        // the wave wait for the request it has just made).
        Grp ga, gb;
        fetch(gi, ga);
        // work's stores, into an empty range: the loop is entered with the
        // memory operations in flight that its back edge has, so the wait
        // for a group's loads need not also wait for the last store
        {
            float z[VEC] = {};
            const rsrc_t none = group_rsrc<T>(a.dx, 0, 0, a.lddx, H);
            bstore_chunk<VEC>((T *)nullptr, none, 0u, z);
            if constexpr (ADD) bstore_chunk<VEC>((T *)nullptr, none, 0u, z);
        }
        while (gi * RPW < N) {
            fetch(gi + gstep, gb);
            work(ga, gi);
            gi += gstep;
            if (gi * RPW >= N) break;
            fetch(gi + gstep, ga);
            work(gb, gi);
            gi += gstep;
        }
    } else {
        for (; gi * RPW < N; gi += gstep) {
            Grp cur;
            fetch(gi, cur);
            work(cur, gi);
        }
    }

    // Partial rows: slot (wave, seg) parks its accumulators in LDS; then
    // each column's SLOTS values are added by one segment of SLOTS lanes
    // with the fixed segment-sum tree (64/SLOTS columns per wave and pass).
    constexpr int CPW = 64 / SLOTS;
    static_assert(SLOTS == 8 || SLOTS == 16 || SLOTS == 32, "slot count");
    const int slot = wave * RPW + seg;
#pragma unroll
    for (int p = 0; p < (LN ? 2 : 1); ++p) {
        const float *src = p == 0 ? adg : adb;
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[slot * SPAN + sl * VEC + k] = src[k];
        __syncthreads();
        float *dst = a.part + (int64_t)p * partial_stride(gridDim.x) * H;
        for (int c0 = wave * CPW; c0 < H; c0 += WPG * CPW) {   // wave-uniform
            const int fc = c0 + lane / SLOTS;
            const float v = fc < H ? acc[(lane % SLOTS) * SPAN + fc] : 0.0f;
            const float t = seg_sum<SLOTS>(v);
            if (lane % SLOTS == 0 && fc < H) {
                if constexpr (FINAL) store_one((W *)(p == 0 ? a.dgamma : a.dbeta) + fc, t);
                else dst[partial_index(blockIdx.x, gridDim.x, H, fc)] = t;
            }
        }
        __syncthreads();
    }
}

}  // namespace rn
