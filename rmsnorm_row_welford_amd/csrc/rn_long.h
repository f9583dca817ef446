// Rows longer than the register-resident plans reach (16-byte path: above
// 16384 elements; element-wise path: above 8192).
//
// One 1024-thread workgroup owns a row at a time and walks it in segments of
// 1024*VEC elements, lane l holding chunk [(s*1024 + l)*VEC, +VEC) of
// segment s (coalesced 16-byte accesses, as in the register plans).  Each
// row is passed over twice: the first pass reads the row from HBM and forms
// the statistics, the second forms the outputs.  These are the pages'
// two-pass designs for rows wider than one tile ("Write Triton Layernorm
// Kernel", Required reasoning process, the loop over column blocks for
// large H; "Write Triton Fused Add Rmsnorm Kernel", Required reasoning
// process, the two-pass variant; "Write Cuda Layernorm Kernel", Kernel
// design rules, the stride loop).  Between the two passes the row stays on
// chip where it fits: its first segments in registers, the next ones in LDS
// (the raw chunks of x, and of the residual or dy, at the same place for the
// same lane, so no lane reads what another wrote and no barrier is needed).
// Otherwise the second pass reads it again from global memory.
//
// Forward statistics, in the read pass of the row (held on chip or read
// twice): RMSNorm and the fused op sum the squares; LayerNorm shifts the
// values by the row's first element, and each lane forms the exact mean and
// M2 of each of its chunks and merges them into a running (count, mean, M2)
// with the parallel merge ("Write Cuda Layernorm Kernel", Required
// reasoning process, the Welford merge formula); the 1024 lanes' states are
// combined by the multi-way form of the same merge:
// mean = sum(n_l m_l)/H, M2 = sum(M2_l + n_l (m_l - mean)^2).  The
// denominator is always H.  A row held on chip is therefore not walked a
// second time for its M2: the statistics overlap the row's loads.
//
// Backward: the first pass forms x_hat, g = dy*gamma and the row sums of g
// and g*x_hat, the second pass forms dx.  With partial rows (rows of up to
// 32 elements per lane, when N makes them pay) a persistent workgroup also
// adds dy*x_hat and dy into per-lane accumulators that become its partial
// row, and caches x and dy in LDS when they fit.  Otherwise the kernel
// writes dx, one row per workgroup held on chip as far as registers and LDS
// go, and then takes its share of the column tiles that form dgamma/dbeta
// from x and dy (colsum_tiles).
#pragma once

#include "rn_kernels.h"

namespace rn {

constexpr int kLongThreads = 1024;
// The backward's per-lane dgamma/dbeta accumulators: 32 elements per lane.
static_assert(kLongAccMaxH == 32 * kLongThreads, "accumulators for 32 elements per lane");
// Segments whose loads are issued together.
#ifndef RN_LONG_UNROLL
#define RN_LONG_UNROLL 4
#endif
// Segments whose parameters the forward's output pass requests together.
#ifndef RN_LONG_OUT_GROUP
#define RN_LONG_OUT_GROUP 2
#endif

// Sum over the 16 waves of a 1024-thread workgroup; every lane gets the same
// bits.  `red` holds two slots of 16 floats used in turn (a slot is written
// again only after every wave has passed the barrier of the sum in between,
// so after every wave has read it).
__device__ __forceinline__ float block_sum16(float v, float *red, int &parity) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63;
    float *slot = red + parity * 16;
    if (lane == 0) slot[wave_id_uniform()] = v;
    __syncthreads();
    const float t = wave_sum(lane < 16 ? slot[lane] : 0.0f);
    parity ^= 1;
    return t;
}

// A raw chunk in LDS: lane-private slots, stored and loaded whole.
template <class T, int VEC>
__device__ __forceinline__ void lds_put(unsigned char *p, const RawChunk<T, VEC> &c) {
    if constexpr (VEC * sizeof(T) == 16) *(u32x4 *)p = __builtin_bit_cast(u32x4, c.v);
    else if constexpr (VEC * sizeof(T) == 4) *(uint32_t *)p = __builtin_bit_cast(uint32_t, c.v);
    else *(uint16_t *)p = (uint16_t)c.v;
}
template <class T, int VEC>
__device__ __forceinline__ void lds_get(const unsigned char *p, RawChunk<T, VEC> &c) {
    if constexpr (VEC * sizeof(T) == 16) c.v = __builtin_bit_cast(decltype(c.v), *(const u32x4 *)p);
    else if constexpr (VEC * sizeof(T) == 4)
        c.v = __builtin_bit_cast(decltype(c.v), *(const uint32_t *)p);
    else c.v = *(const uint16_t *)p;
}

// Bytes of one row of T in the LDS cache (rounded to 16).
__host__ __device__ inline uint32_t long_row_pad(int H, int esize) {
    return ((uint32_t)H * (uint32_t)esize + 15u) & ~15u;
}

// Raw chunks of each input that the on-chip forward keeps in registers:
// 32 registers' worth (16 for each of the fused op's two inputs).
template <class T, int VEC, int OP>
constexpr int fwd_reg_segs() {
    constexpr int words = (VEC * (int)sizeof(T) + 3) / 4;
    return (OP == OP_FUSED ? 16 : 32) / words;
}

// Output of one chunk of the forward: y (and h for the fused op).  v: the
// chunk's values (x, or x + residual in fp32).
template <class T, class W, int VEC, int OP>
__device__ __forceinline__ void fwd_long_out(const float *v, const RawChunk<W, VEC> &cg,
                                             const RawChunk<W, VEC> &cb, float pivot,
                                             float ms, float rstd, rsrc_t ry, rsrc_t rh,
                                             uint32_t off) {
    // h in the same pass as y; every input of the row was read before, so
    // h may alias x or the residual
    if constexpr (OP == OP_FUSED) bstore_chunk<VEC>((T *)nullptr, rh, off, v);
    float out[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        if constexpr (OP == OP_LN) {
            const float d = (v[k] - pivot) - ms;   // x - mean
            out[k] = __builtin_fmaf(d * rstd, cg.get(k), cb.get(k));
        } else {
            out[k] = (v[k] * rstd) * cg.get(k);
        }
    }
    bstore_chunk<VEC>((T *)nullptr, ry, off, out);
}

// Forward of rows held on chip: segments [0, R) of each input in registers,
// the next `nlds` in LDS (LSEG), so every input element crosses HBM once.
// Rows that half the register budget holds (R below fwd_reg_segs) leave
// room for two workgroups per CU: one loads its row while the other reduces
// and stores.
template <class T, class W, int VEC, int OP, int R, bool LSEG>
__global__ __launch_bounds__(kLongThreads, (R < fwd_reg_segs<T, VEC, OP>()) ? 8 : 1)
void fwd_onchip_kernel(const FwdArgs a, int nlds) {
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    constexpr int U = RN_LONG_UNROLL;
    // float32 parameters beside 16-bit rows take twice the registers
    constexpr int G = sizeof(W) > sizeof(T) ? 1 : RN_LONG_OUT_GROUP;
    static_assert(R % G == 0, "whole output groups");
    constexpr int NIN = (OP == OP_FUSED) ? 2 : 1;
    constexpr int SPAN = kLongThreads * VEC;
    constexpr int ES = (int)sizeof(T);
    extern __shared__ f32x4 lds_cache[];
    __shared__ float red[2 * 16];
    unsigned char *lds = (unsigned char *)lds_cache;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int nseg = (H + SPAN - 1) / SPAN;   // at most R + nlds
    const uint32_t nb = (uint32_t)H * (uint32_t)ES;
    const uint32_t lin = (uint32_t)nlds * (uint32_t)(SPAN * ES);   // LDS bytes per input
    const rsrc_t rg = make_rsrc(a.gamma, (uint32_t)H * (uint32_t)sizeof(W));
    const rsrc_t rbt = make_rsrc(a.beta ? a.beta : a.gamma,
                                 a.beta ? (uint32_t)H * (uint32_t)sizeof(W) : 0u);
    // first element of the lane's chunk in segment s, and its LDS slot
    auto el = [&](int s) { return s * SPAN + tid * VEC; };
    auto lslot = [&](int s) { return (uint32_t)(((s - R) * SPAN + tid * VEC) * ES); };
    int parity = 0;

    for (int64_t row = blockIdx.x; row < a.N; row += gridDim.x) {
        const rsrc_t rx = make_rsrc((const T *)a.x + row * a.ldx, nb);
        const rsrc_t rr =
            make_rsrc(OP == OP_FUSED ? (const T *)a.res + row * a.ldr : (const T *)a.x,
                      OP == OP_FUSED ? nb : 0u);
        // ---- pass 1: every load of the row, the LDS copies and the first sums
        Raw reg[NIN][R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            reg[0][u].template bload<RN_LOAD_AUX>(rx, el(u) * ES);
            if constexpr (OP == OP_FUSED) reg[1][u].template bload<RN_LOAD_AUX>(rr, el(u) * ES);
        }
        float pivot = 0.0f;
        if constexpr (OP == OP_LN) {
            RawChunk<T, 1> p0;
            p0.template bload<0>(rx, 0);
            pivot = p0.get(0);
        }
        // LayerNorm: the lane's running (count, mean, M2) about the pivot,
        // each chunk's exact two-pass mean and M2 merged in as it arrives
        // (the parallel merge); the others: the sum of squares
        float s1 = 0.0f;
        float ln_n = 0.0f, ln_m = 0.0f, ln_q = 0.0f;
        auto add1 = [&](const float *v) {
            if constexpr (OP == OP_LN) {
                float uu[VEC], sm = 0.0f;
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    uu[k] = v[k] - pivot;
                    sm += uu[k];
                }
                const float mc = sm * (1.0f / (float)VEC);
                float m2c = 0.0f;
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const float d = uu[k] - mc;
                    m2c = __builtin_fmaf(d, d, m2c);
                }
                const float n1 = ln_n + (float)VEC;
                const float f = (float)VEC / n1;
                const float dl = mc - ln_m;
                ln_m = __builtin_fmaf(dl, f, ln_m);
                ln_q += m2c + dl * dl * (ln_n * f);
                ln_n = n1;
            } else {
#pragma unroll
                for (int k = 0; k < VEC; ++k) s1 = __builtin_fmaf(v[k], v[k], s1);
            }
        };
        auto widen = [&](const Raw &c0, const Raw &c1, float *v) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                v[k] = c0.get(k);
                if constexpr (OP == OP_FUSED) v[k] += c1.get(k);
            }
        };
        // LDS segments, a group of U at a time, the next group requested
        // before the current one is parked
        if constexpr (LSEG) {
            Raw ca[U][NIN], cb[U][NIN];
            auto request = [&](Raw (&c)[U][NIN], int s0) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    c[u][0].template bload<RN_LOAD_AUX>(rx, el(s0 + u) * ES);
                    if constexpr (OP == OP_FUSED)
                        c[u][1].template bload<RN_LOAD_AUX>(rr, el(s0 + u) * ES);
                }
            };
            auto park = [&](Raw (&c)[U][NIN], int s0) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (el(s0 + u) < H) {   // chunks are whole (H is a multiple of VEC)
#pragma unroll
                        for (int i = 0; i < NIN; ++i)
                            lds_put<T, VEC>(lds + i * lin + lslot(s0 + u), c[u][i]);
                        float v[VEC];
                        widen(c[u][0], c[u][NIN - 1], v);
                        add1(v);
                    }
                }
            };
            // Segments past R always exist here.  The register segments are
            // summed while the first LDS group is in flight rather than after
            // the last one is parked, so their arithmetic overlaps the loads.
            request(ca, R);
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if (el(u) < H) {
                    float v[VEC];
                    widen(reg[0][u], reg[NIN - 1][u], v);
                    add1(v);
                }
            }
            for (int s0 = R; s0 < nseg; s0 += 2 * U) {
                if (s0 + U < nseg) request(cb, s0 + U);
                park(ca, s0);
                if (s0 + U >= nseg) break;
                if (s0 + 2 * U < nseg) request(ca, s0 + 2 * U);
                park(cb, s0 + U);
            }
        } else {
#pragma unroll
            for (int u = 0; u < R; ++u) {
                if (el(u) < H) {
                    float v[VEC];
                    widen(reg[0][u], reg[NIN - 1][u], v);
                    add1(v);
                }
            }
        }
        // keep the held chunks packed across the reductions (widened again
        // where used) rather than as float32 copies
        auto repack = [&]() {
#pragma unroll
            for (int u = 0; u < R; ++u)
#pragma unroll
                for (int i = 0; i < NIN; ++i) opaque(reg[i][u].v);
        };
        repack();
        float ms = 0.0f, var;
        if constexpr (OP == OP_LN) {
            // multi-way merge of the lanes' states (about the pivot)
            ms = block_sum16(ln_n * ln_m, red, parity) * a.inv_H;
            const float dm = ln_m - ms;
            var = block_sum16(__builtin_fmaf(ln_n * dm, dm, ln_q), red, parity) * a.inv_H;
        } else {
            var = block_sum16(s1, red, parity) * a.inv_H;
        }
        const float rstd = rsqrt_pos(var + a.eps);
        if (tid == 0) {
            if constexpr (OP == OP_LN) {
                if (a.mean) a.mean[row] = pivot + ms;
            }
            if (a.rstd) a.rstd[row] = rstd;
        }
        // ---- pass 2: outputs, parameters requested G segments at a time
        const rsrc_t ry = make_rsrc((T *)a.y + row * a.ldy, nb);
        const rsrc_t rh = make_rsrc(OP == OP_FUSED ? (T *)a.h + row * a.ldh : (T *)a.y,
                                    OP == OP_FUSED ? nb : 0u);
#pragma unroll
        for (int u0 = 0; u0 < R; u0 += G) {
            if (u0 < nseg) {
                RawW cg[G], cb[G];
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    const int woff = el(u0 + u) * (int)sizeof(W);
                    cg[u].template bload<0>(rg, woff);
                    if constexpr (OP == OP_LN) cb[u].template bload<0>(rbt, woff);
                }
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    float v[VEC];
                    widen(reg[0][u0 + u], reg[NIN - 1][u0 + u], v);
                    fwd_long_out<T, W, VEC, OP>(v, cg[u], cb[u], pivot, ms, rstd, ry, rh,
                                                (uint32_t)(el(u0 + u) * ES));
                }
            }
        }
        if constexpr (LSEG) for (int s0 = R; s0 < nseg; s0 += G) {
            Raw c[G][NIN];
            RawW cg[G], cb[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int woff = el(s0 + u) * (int)sizeof(W);
                cg[u].template bload<0>(rg, woff);
                if constexpr (OP == OP_LN) cb[u].template bload<0>(rbt, woff);
#pragma unroll
                for (int i = 0; i < NIN; ++i) {
                    if (el(s0 + u) < H) lds_get<T, VEC>(lds + i * lin + lslot(s0 + u), c[u][i]);
                    else c[u][i].zero();
                }
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                float v[VEC];
                widen(c[u][0], c[u][NIN - 1], v);
                fwd_long_out<T, W, VEC, OP>(v, cg[u], cb[u], pivot, ms, rstd, ry, rh,
                                            (uint32_t)(el(s0 + u) * ES));
            }
        }
    }
}

// Forward of rows too long to hold on chip: x (and the residual) are read
// twice, the statistics in one pass by the chunk-wise parallel merge.
template <class T, class W, int VEC, int OP>
__global__ __launch_bounds__(kLongThreads) void fwd_long_kernel(const FwdArgs a) {
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    constexpr int U = RN_LONG_UNROLL;
    constexpr int NIN = (OP == OP_FUSED) ? 2 : 1;
    constexpr int SPAN = kLongThreads * VEC;
    __shared__ float red[2 * 16];
    const int tid = threadIdx.x;
    const int H = a.H;
    const int nseg = (H + SPAN - 1) / SPAN;
    const uint32_t nb = (uint32_t)H * (uint32_t)sizeof(T);
    const rsrc_t rg = make_rsrc(a.gamma, (uint32_t)H * (uint32_t)sizeof(W));
    const rsrc_t rbt = make_rsrc(a.beta ? a.beta : a.gamma,
                                 a.beta ? (uint32_t)H * (uint32_t)sizeof(W) : 0u);
    int parity = 0;

    for (int64_t row = blockIdx.x; row < a.N; row += gridDim.x) {
        const rsrc_t rx = make_rsrc((const T *)a.x + row * a.ldx, nb);
        const rsrc_t rr =
            make_rsrc(OP == OP_FUSED ? (const T *)a.res + row * a.ldr : (const T *)a.x,
                      OP == OP_FUSED ? nb : 0u);
        // LayerNorm pivot: the row's first element (every lane loads it)
        float pivot = 0.0f;
        if constexpr (OP == OP_LN) {
            RawChunk<T, 1> p0;
            p0.template bload<0>(rx, 0);
            pivot = p0.get(0);
        }
        // ---- pass 1: statistics
        float ln_n = 0.0f, ln_m = 0.0f, ln_q = 0.0f, q = 0.0f;
        for (int s0 = 0; s0 < nseg; s0 += U) {
            Raw cx[U][NIN];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t off = (uint32_t)(((s0 + u) * SPAN + tid * VEC) * (int)sizeof(T));
                cx[u][0].template bload<RN_LOAD_AUX>(rx, off);
                if constexpr (OP == OP_FUSED) cx[u][1].template bload<RN_LOAD_AUX>(rr, off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (s0 + u) * SPAN + tid * VEC;
                if constexpr (OP == OP_LN) {
                    if (e0 < H) {
                        // exact two-pass mean and M2 of the chunk, then the
                        // parallel merge into the lane's running state
                        float uu[VEC], sm = 0.0f;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            uu[k] = cx[u][0].get(k) - pivot;
                            sm += uu[k];
                        }
                        const float mc = sm * (1.0f / (float)VEC);
                        float m2c = 0.0f;
#pragma unroll
                        for (int k = 0; k < VEC; ++k) {
                            const float d = uu[k] - mc;
                            m2c = __builtin_fmaf(d, d, m2c);
                        }
                        const float n1 = ln_n + (float)VEC;
                        const float f = (float)VEC / n1;
                        const float dl = mc - ln_m;
                        ln_m = __builtin_fmaf(dl, f, ln_m);
                        ln_q += m2c + dl * dl * (ln_n * f);
                        ln_n = n1;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) {
                        float v = cx[u][0].get(k);
                        if constexpr (OP == OP_FUSED) v += cx[u][1].get(k);
                        q = __builtin_fmaf(v, v, q);
                    }
                }
            }
        }
        float ms = 0.0f, var;
        if constexpr (OP == OP_LN) {
            // multi-way merge of the lanes' states (about the pivot)
            ms = block_sum16(ln_n * ln_m, red, parity) * a.inv_H;
            const float dm = ln_m - ms;
            var = block_sum16(__builtin_fmaf(ln_n * dm, dm, ln_q), red, parity) * a.inv_H;
        } else {
            var = block_sum16(q, red, parity) * a.inv_H;
        }
        const float rstd = rsqrt_pos(var + a.eps);
        if (tid == 0) {
            if constexpr (OP == OP_LN) {
                if (a.mean) a.mean[row] = pivot + ms;
            }
            if (a.rstd) a.rstd[row] = rstd;
        }
        // ---- pass 2: outputs, the row read again
        const rsrc_t ry = make_rsrc((T *)a.y + row * a.ldy, nb);
        const rsrc_t rh = make_rsrc(OP == OP_FUSED ? (T *)a.h + row * a.ldh : (T *)a.y,
                                    OP == OP_FUSED ? nb : 0u);
        for (int s0 = 0; s0 < nseg; s0 += U) {
            Raw cx[U][NIN];
            RawW cg[U], cb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (s0 + u) * SPAN + tid * VEC;
                const uint32_t off = (uint32_t)(e0 * (int)sizeof(T));
                cx[u][0].template bload<RN_LOAD_AUX>(rx, off);
                if constexpr (OP == OP_FUSED) cx[u][1].template bload<RN_LOAD_AUX>(rr, off);
                const uint32_t woff = (uint32_t)(e0 * (int)sizeof(W));
                cg[u].template bload<0>(rg, woff);
                if constexpr (OP == OP_LN) cb[u].template bload<0>(rbt, woff);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    v[k] = cx[u][0].get(k);
                    if constexpr (OP == OP_FUSED) v[k] += cx[u][1].get(k);
                }
                // h is stored from values this lane read in this same pass
                fwd_long_out<T, W, VEC, OP>(
                    v, cg[u], cb[u], pivot, ms, rstd, ry, rh,
                    (uint32_t)(((s0 + u) * SPAN + tid * VEC) * (int)sizeof(T)));
            }
        }
    }
}

// dx of one chunk of the backward (and, for the fused op, dh_in added and
// the second copy stored).  LayerNorm: dx = rstd*g + (x_hat*k2 + k1) with
// k2 = -c2*rstd, k1 = -c1*rstd; RMSNorm: dx = (g - x_hat*c2)*rstd.
template <class T, class W, int VEC, bool LN, bool ADD>
__device__ __forceinline__ void bwd_long_dx(const RawChunk<T, VEC> &cx,
                                            const RawChunk<T, VEC> &cd,
                                            const RawChunk<W, VEC> &cg,
                                            const RawChunk<T, VEC> &ca, bool has_add,
                                            float mu, float s, float c2, float k1, float k2,
                                            rsrc_t rdx, rsrc_t rdx2, uint32_t off) {
    float dx[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        const float xhat = (cx.get(k) - mu) * s;
        const float t = cd.get(k) * cg.get(k);
        if constexpr (LN) dx[k] = __builtin_fmaf(t, s, __builtin_fmaf(xhat, k2, k1));
        else dx[k] = __builtin_fmaf(-xhat, c2, t) * s;
        if constexpr (ADD) {
            if (has_add) dx[k] += ca.get(k);
        }
    }
    bstore_chunk<VEC>((T *)nullptr, rdx, off, dx);
    if constexpr (ADD) bstore_chunk<VEC>((T *)nullptr, rdx2, off, dx);
}

// Raw chunks of x and of dy that the backward without accumulators keeps in
// registers: 32 registers' worth of each (24 beside float32 parameters).
template <class T, class W, int VEC>
constexpr int bwd_reg_segs() {
    return (sizeof(W) > sizeof(T) ? 24 : 32) / ((VEC * (int)sizeof(T) + 3) / 4);
}

// Backward without accumulators: dx, one row per workgroup, held on chip as
// far as it fits (segments [0, R) of x and dy in registers, the next `nlds`
// in LDS; the rest are read again by the dx pass), then dgamma/dbeta by
// column tiles (colsum_tiles, CL lanes across each tile).  ADD: the fused
// add+RMSNorm backward (a.add, if set, is added to dx; a.dx2, if set,
// receives dx too).
template <class T, class W, int VEC, bool LN, bool ADD, int CL>
__global__ __launch_bounds__(kLongThreads) void bwd_onchip_kernel(const BwdArgs a, int nlds) {
    static_assert(!(LN && ADD), "the residual variant is RMSNorm's");
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    constexpr int R = bwd_reg_segs<T, W, VEC>();
    // segments per group past the registers, and register segments whose
    // parameters come together (one with float32 parameters beside 16-bit
    // rows: twice the registers)
    constexpr int U = sizeof(W) > sizeof(T) ? 1 : 2;
    constexpr int G = U;
    static_assert(R % G == 0, "whole parameter groups");
    constexpr int SPAN = kLongThreads * VEC;
    constexpr int ES = (int)sizeof(T);
    extern __shared__ f32x4 lds_cache[];
    __shared__ float red[2 * 16];
    unsigned char *lds = (unsigned char *)lds_cache;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int nseg = (H + SPAN - 1) / SPAN;
    const int lend = R + nlds;   // segments from here on are read twice
    const uint32_t nb = (uint32_t)H * (uint32_t)ES;
    const uint32_t lin = (uint32_t)nlds * (uint32_t)(SPAN * ES);   // LDS bytes of x; dy follows
    const rsrc_t rg = make_rsrc(a.gamma, (uint32_t)H * (uint32_t)sizeof(W));
    const T *addb = (const T *)a.add;
    const bool has_add = ADD && addb != nullptr;
    auto el = [&](int sgm) { return sgm * SPAN + tid * VEC; };
    auto lslot = [&](int sgm) { return (uint32_t)(((sgm - R) * SPAN + tid * VEC) * ES); };
    auto woff = [&](int sgm) { return el(sgm) * (int)sizeof(W); };
    int parity = 0;

    for (int64_t row = blockIdx.x; row < a.N; row += gridDim.x) {
        const rsrc_t rx = make_rsrc((const T *)a.x + row * a.ldx, nb);
        const rsrc_t rdy = make_rsrc((const T *)a.dy + row * a.lddy, nb);
        const float mu = LN ? a.mean[row] : 0.0f;
        const float s = a.rstd[row];
        float sg = 0.0f, sgx = 0.0f;
        auto add1 = [&](const Raw &cx, const Raw &cd, const RawW &cg) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float xhat = (cx.get(k) - mu) * s;
                const float gv = cd.get(k) * cg.get(k);
                sg += gv;
                sgx = __builtin_fmaf(gv, xhat, sgx);
            }
        };
        // ---- pass 1: the row sums (and the LDS copies)
        Raw rgx[R], rgd[R];
#pragma unroll
        for (int u = 0; u < R; ++u) {
            rgx[u].template bload<RN_LOAD_AUX>(rx, el(u) * ES);
            rgd[u].template bload<RN_LOAD_AUX>(rdy, el(u) * ES);
        }
        for (int s0 = R; s0 < nseg; s0 += U) {
            Raw cx[U], cd[U];
            RawW cg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                cx[u].template bload<RN_LOAD_AUX>(rx, el(s0 + u) * ES);
                cd[u].template bload<RN_LOAD_AUX>(rdy, el(s0 + u) * ES);
                cg[u].template bload<0>(rg, woff(s0 + u));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (el(s0 + u) < H) {
                    if (s0 + u < lend) {
                        lds_put<T, VEC>(lds + lslot(s0 + u), cx[u]);
                        lds_put<T, VEC>(lds + lin + lslot(s0 + u), cd[u]);
                    }
                    add1(cx[u], cd[u], cg[u]);
                }
            }
        }
#pragma unroll
        for (int u0 = 0; u0 < R; u0 += G) {
            if (u0 < nseg) {
                RawW cg[G];
#pragma unroll
                for (int u = 0; u < G; ++u) cg[u].template bload<0>(rg, woff(u0 + u));
#pragma unroll
                for (int u = 0; u < G; ++u)
                    if (el(u0 + u) < H) add1(rgx[u0 + u], rgd[u0 + u], cg[u]);
            }
        }
        // keep the held chunks packed across the reductions
#pragma unroll
        for (int u = 0; u < R; ++u) {
            opaque(rgx[u].v);
            opaque(rgd[u].v);
        }
        const float c1 = LN ? block_sum16(sg, red, parity) * a.inv_H : 0.0f;
        const float c2 = block_sum16(sgx, red, parity) * a.inv_H;
        const float k2 = -c2 * s, k1 = -c1 * s;
        // ---- pass 2: dx
        const rsrc_t rdx = make_rsrc((T *)a.dx + row * a.lddx, nb);
        const rsrc_t rad = make_rsrc(has_add ? addb + row * a.ldadd : (const T *)a.x,
                                     has_add ? nb : 0u);
        const bool two = ADD && a.dx2 != nullptr;
        const rsrc_t rdx2 = make_rsrc(two ? (T *)a.dx2 + row * a.lddx2 : (T *)a.dx,
                                      two ? nb : 0u);
#pragma unroll
        for (int u0 = 0; u0 < R; u0 += G) {
            if (u0 < nseg) {
                RawW cg[G];
                Raw ca[G];
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    cg[u].template bload<0>(rg, woff(u0 + u));
                    if constexpr (ADD) ca[u].template bload<RN_LOAD_AUX>(rad, el(u0 + u) * ES);
                }
#pragma unroll
                for (int u = 0; u < G; ++u)
                    bwd_long_dx<T, W, VEC, LN, ADD>(rgx[u0 + u], rgd[u0 + u], cg[u], ca[u],
                                                    has_add, mu, s, c2, k1, k2, rdx, rdx2,
                                                    (uint32_t)(el(u0 + u) * ES));
            }
        }
        for (int s0 = R; s0 < nseg; s0 += U) {
            Raw cx[U], cd[U], ca[U];
            RawW cg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int sgm = s0 + u;
                if (sgm < lend) {
                    if (el(sgm) < H) {
                        lds_get<T, VEC>(lds + lslot(sgm), cx[u]);
                        lds_get<T, VEC>(lds + lin + lslot(sgm), cd[u]);
                    } else {
                        cx[u].zero();
                        cd[u].zero();
                    }
                } else {
                    cx[u].template bload<RN_LOAD_AUX>(rx, el(sgm) * ES);
                    cd[u].template bload<RN_LOAD_AUX>(rdy, el(sgm) * ES);
                }
                cg[u].template bload<0>(rg, woff(sgm));
                if constexpr (ADD) ca[u].template bload<RN_LOAD_AUX>(rad, el(sgm) * ES);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                bwd_long_dx<T, W, VEC, LN, ADD>(cx[u], cd[u], cg[u], ca[u], has_add, mu, s, c2,
                                                k1, k2, rdx, rdx2, (uint32_t)(el(s0 + u) * ES));
        }
    }
    colsum_tiles<T, W, VEC, LN, kLongThreads, CL>(a);
}

// Backward with partial rows: a persistent grid whose lanes keep dgamma
// (and dbeta) accumulators for their columns over all the workgroup's rows,
// written at the end as the workgroup's float32 partial row (row-major:
// part[b*H + j], dbeta rows after partial_stride(P)*H floats); rows of at
// most kLongAccMaxH elements.  ADD: as in bwd_onchip_kernel.  `cache`: x
// and dy of the row (two rows of long_row_pad bytes) wait in LDS between
// the passes.
template <class T, class W, int VEC, bool LN, bool ADD>
__global__ __launch_bounds__(kLongThreads) void bwd_long_acc_kernel(const BwdArgs a, int cache) {
    static_assert(!(LN && ADD), "the residual variant is RMSNorm's");
    using Raw = RawChunk<T, VEC>;
    using RawW = RawChunk<W, VEC>;
    // beside the accumulators, two segments in flight (registers)
    constexpr int U = 2;
    constexpr int SPAN = kLongThreads * VEC;
    constexpr int MAXSEG = kLongAccMaxH / SPAN;
    static_assert(MAXSEG % U == 0, "whole segment groups");
    constexpr int EA = MAXSEG * VEC;
    extern __shared__ f32x4 lds_cache[];
    __shared__ float red[2 * 16];
    unsigned char *lds = (unsigned char *)lds_cache;
    const int tid = threadIdx.x;
    const int H = a.H;
    const int nseg = (H + SPAN - 1) / SPAN;
    const uint32_t pad = long_row_pad(H, (int)sizeof(T));
    const uint32_t nb = (uint32_t)H * (uint32_t)sizeof(T);
    const rsrc_t rg = make_rsrc(a.gamma, (uint32_t)H * (uint32_t)sizeof(W));
    const T *addb = (const T *)a.add;
    const bool has_add = ADD && addb != nullptr;
    int parity = 0;

    float adg[EA], adb[LN ? EA : 1];
#pragma unroll
    for (int e = 0; e < EA; ++e) adg[e] = 0.0f;
#pragma unroll
    for (int e = 0; e < (LN ? EA : 1); ++e) adb[e] = 0.0f;

    for (int64_t row = blockIdx.x; row < a.N; row += gridDim.x) {
        const rsrc_t rx = make_rsrc((const T *)a.x + row * a.ldx, nb);
        const rsrc_t rdy = make_rsrc((const T *)a.dy + row * a.lddy, nb);
        const float mu = LN ? a.mean[row] : 0.0f;
        const float s = a.rstd[row];
        float sg = 0.0f, sgx = 0.0f;
        // ---- pass 1: the row sums (and the accumulators, and the LDS copy)
        auto pass1 = [&](const int s0) {
            Raw cx[U], cd[U];
            RawW cg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (s0 + u) * SPAN + tid * VEC;
                const uint32_t off = (uint32_t)(e0 * (int)sizeof(T));
                cx[u].template bload<RN_LOAD_AUX>(rx, off);
                cd[u].template bload<RN_LOAD_AUX>(rdy, off);
                cg[u].template bload<0>(rg, (uint32_t)(e0 * (int)sizeof(W)));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (s0 + u) * SPAN + tid * VEC;
                if (cache && e0 < H) {
                    const uint32_t off = (uint32_t)(e0 * (int)sizeof(T));
                    lds_put<T, VEC>(lds + off, cx[u]);
                    lds_put<T, VEC>(lds + pad + off, cd[u]);
                }
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const float dyv = cd[u].get(k);
                    const float xhat = (cx[u].get(k) - mu) * s;
                    const float gv = dyv * cg[u].get(k);
                    sg += gv;
                    sgx = __builtin_fmaf(gv, xhat, sgx);
                    const int e = (s0 + u) * VEC + k;   // constant: s0 is unrolled
                    adg[e] = __builtin_fmaf(dyv, xhat, adg[e]);
                    if constexpr (LN) adb[e] += dyv;
                }
            }
        };
#pragma unroll
        for (int s0 = 0; s0 < MAXSEG; s0 += U)
            if (s0 < nseg) pass1(s0);
        const float c1 = LN ? block_sum16(sg, red, parity) * a.inv_H : 0.0f;
        const float c2 = block_sum16(sgx, red, parity) * a.inv_H;
        // LayerNorm: dx = rstd*g + (x_hat*(-c2*rstd) + (-c1*rstd))
        const float k2 = -c2 * s, k1 = -c1 * s;
        // ---- pass 2: dx
        const rsrc_t rdx = make_rsrc((T *)a.dx + row * a.lddx, nb);
        const rsrc_t rad = make_rsrc(has_add ? addb + row * a.ldadd : (const T *)a.x,
                                     has_add ? nb : 0u);
        const bool two = ADD && a.dx2 != nullptr;
        const rsrc_t rdx2 = make_rsrc(two ? (T *)a.dx2 + row * a.lddx2 : (T *)a.dx,
                                      two ? nb : 0u);
        for (int s0 = 0; s0 < nseg; s0 += U) {
            Raw cx[U], cd[U], ca[ADD ? U : 1];
            RawW cg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e0 = (s0 + u) * SPAN + tid * VEC;
                const uint32_t off = (uint32_t)(e0 * (int)sizeof(T));
                if (cache) {
                    if (e0 < H) {
                        lds_get<T, VEC>(lds + off, cx[u]);
                        lds_get<T, VEC>(lds + pad + off, cd[u]);
                    } else {
                        cx[u].zero();
                        cd[u].zero();
                    }
                } else {
                    cx[u].template bload<RN_LOAD_AUX>(rx, off);
                    cd[u].template bload<RN_LOAD_AUX>(rdy, off);
                }
                cg[u].template bload<0>(rg, (uint32_t)(e0 * (int)sizeof(W)));
                if constexpr (ADD) ca[u].template bload<RN_LOAD_AUX>(rad, off);
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                bwd_long_dx<T, W, VEC, LN, ADD>(
                    cx[u], cd[u], cg[u], ca[ADD ? u : 0], has_add, mu, s, c2, k1, k2, rdx, rdx2,
                    (uint32_t)(((s0 + u) * SPAN + tid * VEC) * (int)sizeof(T)));
        }
    }

    {
        float *pg = a.part + (int64_t)blockIdx.x * H;
        float *pb = a.part + (int64_t)partial_stride(gridDim.x) * H + (int64_t)blockIdx.x * H;
#pragma unroll
        for (int sg_ = 0; sg_ < MAXSEG; ++sg_) {
            const int col = sg_ * SPAN + tid * VEC;
            if (col < H) {
                store_f32s<VEC>(pg + col, adg + sg_ * VEC);
                if constexpr (LN) store_f32s<VEC>(pb + col, adb + sg_ * VEC);
            }
        }
    }
}

// ------------------------------------------------------------- launches --
// Dynamic LDS the cache of `rows` rows of H elements of T needs, or 0 when
// it does not fit in `budget` bytes.
inline int long_cache_bytes(int H, int esize, int rows, int budget) {
    const int64_t b = (int64_t)rows * long_row_pad(H, esize);
    return b <= budget ? (int)b : 0;
}

// Allow kernel K up to `bytes` of dynamic LDS (once per kernel).
template <auto K>
inline void allow_lds(int bytes) {
    static std::atomic<int> done{0};
    if (bytes > 0 && done.load(std::memory_order_relaxed) < bytes) {
        if (hipFuncSetAttribute((const void *)K, hipFuncAttributeMaxDynamicSharedMemorySize,
                                bytes) == hipSuccess)
            done.store(bytes, std::memory_order_relaxed);
    }
}

template <class T, class W, int VEC, int OP>
hipError_t launch_fwd_long_op(const FwdArgs &a, hipStream_t s) {
    constexpr int NIN = (OP == OP_FUSED) ? 2 : 1;
    constexpr int R = fwd_reg_segs<T, VEC, OP>();
    constexpr int SPAN = kLongThreads * VEC;
    const int nseg = (a.H + SPAN - 1) / SPAN;
    const int nlds = nseg > R ? nseg - R : 0;
    const int64_t lds = (int64_t)nlds * NIN * SPAN * (int64_t)sizeof(T);
    const int64_t grid = a.N < (1 << 20) ? a.N : (1 << 20);
    if (lds <= long_lds_budget()) {
        // the row fits in registers (and LDS): one read
        constexpr int RH = R / 2;
        if (nseg <= RH) {
            hipLaunchKernelGGL((fwd_onchip_kernel<T, W, VEC, OP, RH, false>),
                               dim3((unsigned)grid), dim3(kLongThreads), 0, s, a, 0);
        } else if (nlds == 0) {
            hipLaunchKernelGGL((fwd_onchip_kernel<T, W, VEC, OP, R, false>),
                               dim3((unsigned)grid), dim3(kLongThreads), 0, s, a, 0);
        } else {
            constexpr auto k = fwd_onchip_kernel<T, W, VEC, OP, R, true>;
            allow_lds<k>((int)lds);
            hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kLongThreads), (unsigned)lds, s,
                               a, nlds);
        }
    } else {
        hipLaunchKernelGGL((fwd_long_kernel<T, W, VEC, OP>), dim3((unsigned)grid),
                           dim3(kLongThreads), 0, s, a);
    }
    return hipGetLastError();
}

template <class T, class W, int VEC>
hipError_t launch_fwd_long(int op, const FwdArgs &a, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_fwd_long_op<T, W, VEC, OP_LN>(a, s);
    case OP_RMS: return launch_fwd_long_op<T, W, VEC, OP_RMS>(a, s);
    default: return launch_fwd_long_op<T, W, VEC, OP_FUSED>(a, s);
    }
}

// The long-row backward's partial-row count: one persistent workgroup per
// CU (at most one row each).
inline int bwd_long_partials(int64_t N, int cus) {
    return (int)(N < cus ? N : cus);
}

// Rows below which the long-row backward's column tiles are 32 lanes wide
// instead of 8: with 8 lanes across, each of the 128 row slots of a tile
// adds only N/128 rows, too little work per workgroup for the loads to
// stay in flight.  Measured at 256 x 131072 (bf16): LN 83 -> 71 us, RMS
// 76 -> 68.5 us (64 lanes: 72.7 and 70 us).
#ifndef RN_LONG_WIDE_TILE_ROWS
#define RN_LONG_WIDE_TILE_ROWS 1024
#endif

// dx, the row held on chip as far as registers and LDS go (LDS less the
// column tiles' static share), then the column tiles
template <class T, class W, int VEC, bool LN, bool ADD, int CL>
hipError_t launch_bwd_onchip(const BwdArgs &a, hipStream_t s) {
    constexpr int R = bwd_reg_segs<T, W, VEC>();
    constexpr int SPAN = kLongThreads * VEC;
    const int nseg = (a.H + SPAN - 1) / SPAN;
    const int pair = 2 * SPAN * (int)sizeof(T);   // LDS bytes of one segment of x and dy
    constexpr int tile_lds =
        ColsumTile<T, VEC, kLongThreads, CL>::LDS_FLOATS * (int)sizeof(float);
    const int budget = long_lds_budget() - tile_lds;
    const int fit = budget > 0 ? budget / pair : 0;
    const int nlds = nseg > R ? (nseg - R < fit ? nseg - R : fit) : 0;
    constexpr auto k = bwd_onchip_kernel<T, W, VEC, LN, ADD, CL>;
    allow_lds<k>(nlds * pair);
    const int64_t rows = a.N < (1 << 20) ? a.N : (1 << 20);
    hipLaunchKernelGGL(k, dim3((unsigned)colsum_grid<VEC>(rows, a.H, CL)),
                       dim3(kLongThreads), (unsigned)(nlds * pair), s, a, nlds);
    return hipGetLastError();
}

template <class T, class W, int VEC, bool LN, bool ADD>
hipError_t launch_bwd_long_t(const BwdArgs &a, int P, bool colsum, void *dg, void *db,
                             hipStream_t s) {
    const int lds = long_cache_bytes(a.H, (int)sizeof(T), 2, long_lds_budget());
    if (!colsum) {
        constexpr auto k = bwd_long_acc_kernel<T, W, VEC, LN, ADD>;
        allow_lds<k>(lds);
        if (P > 0) {
            hipLaunchKernelGGL(k, dim3(P), dim3(kLongThreads), lds, s, a, lds > 0 ? 1 : 0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return launch_bwd2<W>(a.part, P, a.H, LN, dg, db, s);
    }
    if (a.N < RN_LONG_WIDE_TILE_ROWS)
        return launch_bwd_onchip<T, W, VEC, LN, ADD, 32>(a, s);
    return launch_bwd_onchip<T, W, VEC, LN, ADD, 8>(a, s);
}

template <class T, class W, int VEC>
hipError_t launch_bwd_long(bool ln, bool fused, const BwdArgs &a, int P, bool colsum,
                           void *dg, void *db, hipStream_t s) {
    if (ln) return launch_bwd_long_t<T, W, VEC, true, false>(a, P, colsum, dg, db, s);
    if (fused) return launch_bwd_long_t<T, W, VEC, false, true>(a, P, colsum, dg, db, s);
    return launch_bwd_long_t<T, W, VEC, false, false>(a, P, colsum, dg, db, s);
}

}  // namespace rn
