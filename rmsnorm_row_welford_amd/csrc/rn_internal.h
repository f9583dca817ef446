// Internal interface between the C-ABI entry points (rn_api.hip) and the
// kernel translation units (one per direction and storage type).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rn {

enum FwdOp : int { OP_LN = 0, OP_RMS = 1, OP_FUSED = 2 };

// Arguments of one forward call, already validated.  Pointers that a given
// op does not use are NULL.  x and h may be the same buffer (fused op), so
// none of these pointers is restrict.
struct FwdArgs {
    const void *x;
    const void *res;
    const void *gamma;
    const void *beta;
    void *y;
    void *h;
    float *mean;
    float *rstd;
    int64_t ldx, ldr, ldy, ldh;
    int64_t N;
    int H;
    float eps;
    float inv_H;
};

// Arguments of one backward call.  `part` is the float32 partial-row
// workspace: P partial rows of dgamma, then (LN) P of dbeta at
// part + partial_stride(P) * H; short rows store each set column-major,
// long rows row-major (partial_colmajor in rn_kernels.h).
// Fused add+RMSNorm backward extras: `add` (NULL = none) is added to dx,
// and `dx2` (NULL = none) receives a second copy of dx.
struct BwdArgs {
    const void *dy;
    const void *x;
    const void *gamma;
    const float *mean;
    const float *rstd;
    void *dx;
    float *part;
    const void *add;
    void *dx2;
    void *dgamma;   // written by kernel 1 itself when one workgroup holds every row
    void *dbeta;
    int64_t lddy, ldx, lddx, ldadd, lddx2;
    int64_t N;
    int H;
    float inv_H;
};

// Column stride of the partial-row workspace: the P float32 partial rows of
// one parameter are stored column by column, each column padded to a
// multiple of 8 slots.
__host__ __device__ inline int partial_stride(int P) { return (P + 7) & ~7; }

// Longest rows the register-resident backward plans hold: 16-byte vector
// path, element-wise path.  Longer rows walk their row in segments
// (rn_long.h).  The forward's vector-path limit is the widest span of its
// plan list (32768 for 2-byte rows with 2-byte parameters, else 16384).
constexpr int kMaxHiddenReg = 16384;
constexpr int kMaxHiddenRegScalar = 8192;
// Longest row any path takes (4 Mi elements: byte offsets within a row stay
// far below 2^31).
constexpr int kMaxHidden = 1 << 22;
inline bool is_long_row(int64_t H, bool vec) {
    return H > (vec ? kMaxHiddenReg : kMaxHiddenRegScalar);
}
// The long-row backward keeps per-lane dgamma/dbeta accumulators (and so
// writes partial rows) for rows of up to this many elements; longer rows
// always take the column-sum strategy.
constexpr int kLongAccMaxH = 32768;
inline bool bwd_force_colsum(int64_t H, bool vec) {
    return is_long_row(H, vec) && H > kLongAccMaxH;
}
// Dynamic LDS a long-row workgroup may use on the current device for its row
// cache (the device's per-workgroup limit less a margin for static LDS).
int long_lds_budget();

// Per storage pair (activations / parameters), one translation unit per
// direction defines:
//   launch_fwd_<S>:   picks the kernel for (op, H, vec) and launches it;
//   bwd_partials_<S>: backward kernel 1's grid (the number of partial rows
//                     P) for a shape, or -1 if H has no plan;
//   launch_bwd_<S>:   the backward: kernel 1 (dx [+ partial rows]) then
//                     kernel 2 (partial rows, or the column sums of the
//                     rows, -> dgamma [, dbeta]).  `P` must equal
//                     bwd_partials_<S>(N, H, vec, cus) and `colsum` must be
//                     bwd_use_colsum(...).  `fused` selects the RMSNorm
//                     kernel variant that also handles a.add and a.dx2 (the
//                     fused add+RMSNorm backward; ln must then be false).
// S: f32, bf16, f16 (parameters in the activation type) and bf16_f32w,
// f16_f32w (float32 parameters).
#define RN_DECLARE_STORAGE(S)                                                        \
    hipError_t launch_fwd_##S(int op, const FwdArgs &a, bool vec, int cus,           \
                              hipStream_t s);                                        \
    int bwd_partials_##S(int64_t N, int H, bool vec, int cus);                      \
    hipError_t launch_bwd_##S(bool ln, bool fused, const BwdArgs &a, bool vec,       \
                              int cus, int P, bool colsum, void *dgamma, void *dbeta, \
                              hipStream_t s);
RN_DECLARE_STORAGE(f32)
RN_DECLARE_STORAGE(bf16)
RN_DECLARE_STORAGE(f16)
RN_DECLARE_STORAGE(bf16_f32w)
RN_DECLARE_STORAGE(f16_f32w)
#undef RN_DECLARE_STORAGE

// Which reduction the backward uses for dgamma/dbeta.  Partial rows cost
// 2*P*H*4 bytes per parameter (written by kernel 1, read by kernel 2); the
// column-sum strategy instead reads x and dy a second time, 2*N*H*e bytes,
// in column tiles that the dx kernel takes after its rows (no second
// launch).  The cheaper one in bytes wins, ties to the column sums
// (RN_BWD_COLSUM_PCT scales the comparison), when the row gives at least
// a quarter of the CUs an 8-chunk column tile.  Measured on MI355X: at
// equal bytes the column sums win by about the second launch (512 x 16384
// RMSNorm: 17.9 -> 16.3 us); when the tiles followed as a kernel of their
// own they paid only with a 2x byte margin.
#ifndef RN_BWD_COLSUM_PCT
#define RN_BWD_COLSUM_PCT 100
#endif
// Rows each team of a backward workgroup may take before the grid grows
// past one workgroup: with a single workgroup its partial row is already
// the column sum, so kernel 1 writes dgamma/dbeta itself and the backward
// is one launch (the few-row, latency-bound regime).
#ifndef RN_BWD_DECODE_ROWS
#define RN_BWD_DECODE_ROWS 4
#endif

inline bool bwd_use_colsum(int64_t N, int H, int e, int P, bool ln, int cus) {
    if (N <= 0 || P <= 0) return false;
    const int cols_per_tile = 8 * (16 / e);
    if (H / cols_per_tile < cus / 4) return false;
    const int64_t partial = (int64_t)8 * P * (ln ? 2 : 1);
    const int64_t reread = (int64_t)2 * N * e;
    return reread * 100 <= partial * RN_BWD_COLSUM_PCT;
}

hipError_t launch_copy(const void *src, void *dst, size_t bytes,
                       hipStream_t s);

// out = a + b over n elements; elem: 0 float32, 1 bfloat16, 2 binary16.
hipError_t launch_add(int elem, const void *a, const void *b, void *out, int64_t n,
                      hipStream_t s);

}  // namespace rn
