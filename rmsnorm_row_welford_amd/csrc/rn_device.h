// Device primitives for the gfx950 row-normalization kernels: vector
// load/store of row chunks with float32 conversion, bfloat16 and binary16
// rounding, and wave64 reductions built from DPP row permutations and row
// broadcasts (ds_swizzle for 32-lane segments).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rn {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bfloat16 values travel as their 16-bit patterns; IEEE binary16 as the
// compiler's _Float16.
typedef uint16_t bf16_bits;
typedef _Float16 f16_t;

// Elements per 16-byte chunk.
template <class T> struct Vec16;
template <> struct Vec16<float> { static constexpr int N = 4; };
template <> struct Vec16<bf16_bits> { static constexpr int N = 8; };
template <> struct Vec16<f16_t> { static constexpr int N = 8; };

// ------------------------------------------------------------------ codec --
__device__ __forceinline__ float bf16_lo(unsigned u) {
    return __uint_as_float(u << 16);
}
__device__ __forceinline__ float bf16_hi(unsigned u) {
    return __uint_as_float(u & 0xffff0000u);
}
// Two float32 -> two bfloat16 (round to nearest even, NaN stays NaN) in one
// v_cvt_pk_bf16_f32; `a` lands in the low half.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16_bits to_bf16(float a) {
    return __builtin_bit_cast(bf16_bits, (__bf16)a);
}
// binary16 <-> float32: widening is exact; narrowing rounds to nearest even
// (the default rounding mode; overflow gives infinity).
__device__ __forceinline__ float f16_lo(unsigned u) {
    return (float)__builtin_bit_cast(f16x2, u)[0];
}
__device__ __forceinline__ float f16_hi(unsigned u) {
    return (float)__builtin_bit_cast(f16x2, u)[1];
}
__device__ __forceinline__ unsigned pack_f16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// 1/sqrt(v) for a normal v > 0 (var + eps; eps is a positive normal float):
// one v_rsq_f32 (about 1 ulp) instead of a correctly rounded square root and
// an IEEE division, a chain of some 30 dependent instructions on every row.
__device__ __forceinline__ float rsqrt_pos(float v) { return __builtin_amdgcn_rsqf(v); }

// ------------------------------------------------------------ chunk I/O --
// Load VEC consecutive elements at p (aligned to VEC elements) as float32.
// NT selects the non-temporal hint for data read exactly once.
template <int VEC, bool NT>
__device__ __forceinline__ void load_chunk(const float *p, float *o) {
    if constexpr (VEC == 4) {
        f32x4 v = NT ? __builtin_nontemporal_load((const f32x4 *)p)
                     : *(const f32x4 *)p;
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    } else {
        static_assert(VEC == 1, "fp32 chunks are 4 or 1 elements");
        o[0] = NT ? __builtin_nontemporal_load(p) : *p;
    }
}
template <int VEC, bool NT>
__device__ __forceinline__ void load_chunk(const bf16_bits *p, float *o) {
    if constexpr (VEC == 8) {
        u32x4 v = NT ? __builtin_nontemporal_load((const u32x4 *)p)
                     : *(const u32x4 *)p;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = bf16_lo(v[k]);
            o[2 * k + 1] = bf16_hi(v[k]);
        }
    } else {
        static_assert(VEC == 1, "bf16 chunks are 8 or 1 elements");
        unsigned u = NT ? __builtin_nontemporal_load(p) : *p;
        o[0] = __uint_as_float(u << 16);
    }
}
template <int VEC, bool NT>
__device__ __forceinline__ void load_chunk(const f16_t *p, float *o) {
    if constexpr (VEC == 8) {
        u32x4 v = NT ? __builtin_nontemporal_load((const u32x4 *)p)
                     : *(const u32x4 *)p;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = f16_lo(v[k]);
            o[2 * k + 1] = f16_hi(v[k]);
        }
    } else {
        static_assert(VEC == 1, "fp16 chunks are 8 or 1 elements");
        o[0] = (float)(NT ? __builtin_nontemporal_load(p) : *p);
    }
}

// ------------------------------------------------------- buffer resources --
// Row I/O goes through raw (untyped) buffer descriptors: a 128-bit SGPR
// resource per row, a byte offset per lane in a VGPR.  The hardware range
// check returns 0 for loads at or past `bytes` and drops such stores, so a
// row's masked chunks need no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, GFX9-family format word
constexpr int AUX_NT = 2;                // non-temporal hint
// Cache-policy bits of the streaming row loads and of the row stores
// (build-time tunable).
#ifndef RN_LOAD_AUX
#define RN_LOAD_AUX AUX_NT
#endif
#ifndef RN_STORE_AUX
#define RN_STORE_AUX AUX_NT
#endif

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes,
                                             kRsrcWord3);
}

// One chunk kept in its storage form (bfloat16 stays packed two per
// register) and widened to float32 on use: gamma/beta for a whole
// persistent loop, and the prefetched chunks of a team's next row.
template <class T, int VEC> struct RawChunk;
template <> struct RawChunk<bf16_bits, 8> {
    u32x4 v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
    __device__ __forceinline__ void gload_nt(const bf16_bits *p) {
        v = __builtin_nontemporal_load((const u32x4 *)p);
    }
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int k) const {
        return (k & 1) ? bf16_hi(v[k >> 1]) : bf16_lo(v[k >> 1]);
    }
};
template <> struct RawChunk<bf16_bits, 1> {
    unsigned v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
    }
    __device__ __forceinline__ void gload_nt(const bf16_bits *p) {
        v = __builtin_nontemporal_load(p);
    }
    __device__ __forceinline__ void zero() { v = 0u; }
    __device__ __forceinline__ float get(int) const { return __uint_as_float(v << 16); }
};
template <> struct RawChunk<f16_t, 8> {
    u32x4 v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
    __device__ __forceinline__ void gload_nt(const f16_t *p) {
        v = __builtin_nontemporal_load((const u32x4 *)p);
    }
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int k) const {
        return (k & 1) ? f16_hi(v[k >> 1]) : f16_lo(v[k >> 1]);
    }
};
template <> struct RawChunk<f16_t, 1> {
    unsigned v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
    }
    __device__ __forceinline__ void gload_nt(const f16_t *p) {
        v = __builtin_nontemporal_load((const uint16_t *)p);
    }
    __device__ __forceinline__ void zero() { v = 0u; }
    __device__ __forceinline__ float get(int) const { return f16_lo(v); }
};
// float32 parameters beside 8-element (2-byte) activation chunks: two
// 16-byte loads per chunk.
template <> struct RawChunk<float, 8> {
    f32x4 v[2];
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v[0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
        v[1] = __builtin_bit_cast(f32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, AUX));
    }
    __device__ __forceinline__ void zero() { v[0] = v[1] = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float get(int k) const { return v[k >> 2][k & 3]; }
};
template <> struct RawChunk<float, 4> {
    f32x4 v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
    __device__ __forceinline__ void gload_nt(const float *p) {
        v = __builtin_nontemporal_load((const f32x4 *)p);
    }
    __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float get(int k) const { return v[k]; }
};
template <> struct RawChunk<float, 1> {
    float v;
    template <int AUX> __device__ __forceinline__ void bload(rsrc_t r, int off) {
        v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX));
    }
    __device__ __forceinline__ void gload_nt(const float *p) { v = __builtin_nontemporal_load(p); }
    __device__ __forceinline__ void zero() { v = 0.f; }
    __device__ __forceinline__ float get(int) const { return v; }
};

// Make a register value opaque to the optimizer (emits no instruction):
// values widened from a packed chunk before this point are then widened
// again after it instead of being kept live as float32 across a reduction.
__device__ __forceinline__ void opaque(u32x4 &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(f32x4 &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(unsigned &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(float &v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(f32x4 (&v)[2]) {
    opaque(v[0]);
    opaque(v[1]);
}

// Store a chunk of VEC float32 values, rounded to the storage type, through
// a buffer resource.
template <int VEC>
__device__ __forceinline__ void bstore_chunk(float *, rsrc_t r, int off, const float *v) {
    if constexpr (VEC == 4) {
        f32x4 w = {v[0], v[1], v[2], v[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), r, off, 0,
                                               RN_STORE_AUX);
    } else {
        static_assert(VEC == 1, "fp32 chunks are 4 or 1 elements");
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v[0]), r, off, 0,
                                              RN_STORE_AUX);
    }
}
template <int VEC>
__device__ __forceinline__ void bstore_chunk(bf16_bits *, rsrc_t r, int off, const float *v) {
    if constexpr (VEC == 8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, RN_STORE_AUX);
    } else {
        static_assert(VEC == 1, "bf16 chunks are 8 or 1 elements");
        __builtin_amdgcn_raw_buffer_store_b16(to_bf16(v[0]), r, off, 0, RN_STORE_AUX);
    }
}

template <int VEC>
__device__ __forceinline__ void bstore_chunk(f16_t *, rsrc_t r, int off, const float *v) {
    if constexpr (VEC == 8) {
        u32x4 w;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack_f16(v[2 * k], v[2 * k + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, RN_STORE_AUX);
    } else {
        static_assert(VEC == 1, "fp16 chunks are 8 or 1 elements");
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (f16_t)v[0]), r,
                                              off, 0, RN_STORE_AUX);
    }
}

// Store one float32 as the storage type.
__device__ __forceinline__ void store_one(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_one(bf16_bits *p, float v) { *p = to_bf16(v); }
__device__ __forceinline__ void store_one(f16_t *p, float v) { *p = (f16_t)v; }

// ------------------------------------------------------ wave reductions --
// DPP controls (GFX9 encoding).
enum : int {
    DPP_QUAD_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
    DPP_ROW_HALF_MIRROR = 0x141,
    DPP_ROW_MIRROR = 0x140,
    DPP_ROW_BCAST15 = 0x142,   // lane 15 of each row feeds the next row
    DPP_ROW_BCAST31 = 0x143,   // lane 31 feeds rows 2 and 3
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                           0xF, 0xF, false));
}

// A DPP read in the rows that ROW_MASK enables; the other rows read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                           ROW_MASK, 0xF, false));
}

// Lane i reads lane i ^ 16 within each half of the wave (ds_swizzle
// bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ float swizzle_xor16(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wave; every lane gets the same bits.
// Each step pairs lanes symmetrically (a+b and b+a round identically), so
// after the four DPP steps all 16 lanes of DPP row k hold the row's sum
// r_k.  Two row broadcasts then finish in the vector unit (no LDS round
// trip): rows 1 and 3 add the row below (r1 + r0, r3 + r2), row 3 adds row
// 1, and lane 63 holds (r3 + r2) + (r1 + r0), the same bits as
// (r0 + r1) + (r2 + r3).  Must be called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    v += dpp<DPP_ROW_MIRROR>(v);
    v += dpp_rows<DPP_ROW_BCAST15, 0xA>(v);
    v += dpp_rows<DPP_ROW_BCAST31, 0xC>(v);
    return lane_value(v, 63);
}

// Two independent sums, interleaved for latency.
__device__ __forceinline__ void wave_sum2(float &a, float &b) {
    a += dpp<DPP_QUAD_XOR1>(a);
    b += dpp<DPP_QUAD_XOR1>(b);
    a += dpp<DPP_QUAD_XOR2>(a);
    b += dpp<DPP_QUAD_XOR2>(b);
    a += dpp<DPP_ROW_HALF_MIRROR>(a);
    b += dpp<DPP_ROW_HALF_MIRROR>(b);
    a += dpp<DPP_ROW_MIRROR>(a);
    b += dpp<DPP_ROW_MIRROR>(b);
    a += dpp_rows<DPP_ROW_BCAST15, 0xA>(a);
    b += dpp_rows<DPP_ROW_BCAST15, 0xA>(b);
    a += dpp_rows<DPP_ROW_BCAST31, 0xC>(a);
    b += dpp_rows<DPP_ROW_BCAST31, 0xC>(b);
    a = lane_value(a, 63);
    b = lane_value(b, 63);
}

// Sum over aligned groups of SEG lanes (8, 16 or 32): the first steps of
// wave_sum; every lane of a group receives the group's sum, with the same
// bits in each lane.  All 64 lanes must be active.
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
    static_assert(SEG == 8 || SEG == 16 || SEG == 32, "segments of 8, 16 or 32 lanes");
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (SEG >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if constexpr (SEG >= 32) v += swizzle_xor16(v);
    return v;
}

__device__ __forceinline__ int wave_id_uniform() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace rn
