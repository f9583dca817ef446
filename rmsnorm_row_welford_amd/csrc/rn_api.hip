// C-ABI entry points of librownorm.so: argument validation, overlap checks,
// plan inputs (vectorizability, CU count) and kernel launches.  All checks
// run before anything is enqueued.
#include <float.h>
#include <math.h>
#include <initializer_list>
#include <mutex>
#include <stdint.h>

#include "../../include/rownorm.h"
#include "../../include/rownorm_bench.h"
#include "rn_internal.h"

using namespace rn;

namespace {

// ------------------------------------------------------- device properties --
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
std::once_flag g_once[kMaxDevices];

int g_lds[kMaxDevices];
std::once_flag g_lds_once[kMaxDevices];

// Compute-unit count of the current device, cached per device.
int current_cus(int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RN_EHIP;
    std::call_once(g_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                                  dev) != hipSuccess)
            n = 0;
        g_cus[dev] = n;
    });
    if (g_cus[dev] <= 0) return RN_EHIP;
    *cus = g_cus[dev];
    return RN_OK;
}

}  // namespace

// Dynamic LDS a long-row workgroup may use: the device's per-workgroup
// limit, less 1 KiB for the kernels' small static LDS (the launches that
// also take column tiles subtract those tiles' share); cached per device.
int rn::long_lds_budget() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(g_lds_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
            n = 0;
        g_lds[dev] = n > 1024 ? n - 1024 : 0;
    });
    return g_lds[dev];
}

namespace {

// Bytes per element of the rn_dtype codes: activations (x, residual, h, y,
// dy, dx, ...) and parameters (gamma, beta, dgamma, dbeta).
bool dtype_ok(int dtype) { return dtype >= RN_F32 && dtype <= RN_F16_F32W; }
size_t elem_size(int dtype) { return dtype == RN_F32 ? 4 : 2; }
size_t param_size(int dtype) { return (dtype == RN_BF16 || dtype == RN_F16) ? 2 : 4; }

hipError_t launch_fwd(int dtype, int op, const FwdArgs &a, bool vec, int cus,
                      hipStream_t s) {
    switch (dtype) {
    case RN_F32: return launch_fwd_f32(op, a, vec, cus, s);
    case RN_BF16: return launch_fwd_bf16(op, a, vec, cus, s);
    case RN_F16: return launch_fwd_f16(op, a, vec, cus, s);
    case RN_BF16_F32W: return launch_fwd_bf16_f32w(op, a, vec, cus, s);
    default: return launch_fwd_f16_f32w(op, a, vec, cus, s);
    }
}

int bwd_partials(int dtype, int64_t N, int H, bool vec, int cus) {
    switch (dtype) {
    case RN_F32: return bwd_partials_f32(N, H, vec, cus);
    case RN_BF16: return bwd_partials_bf16(N, H, vec, cus);
    case RN_F16: return bwd_partials_f16(N, H, vec, cus);
    case RN_BF16_F32W: return bwd_partials_bf16_f32w(N, H, vec, cus);
    default: return bwd_partials_f16_f32w(N, H, vec, cus);
    }
}

hipError_t launch_bwd(int dtype, bool ln, bool fused, const BwdArgs &a, bool vec,
                      int cus, int P, bool colsum, void *dg, void *db, hipStream_t s) {
    switch (dtype) {
    case RN_F32: return launch_bwd_f32(ln, fused, a, vec, cus, P, colsum, dg, db, s);
    case RN_BF16: return launch_bwd_bf16(ln, fused, a, vec, cus, P, colsum, dg, db, s);
    case RN_F16: return launch_bwd_f16(ln, fused, a, vec, cus, P, colsum, dg, db, s);
    case RN_BF16_F32W:
        return launch_bwd_bf16_f32w(ln, fused, a, vec, cus, P, colsum, dg, db, s);
    default: return launch_bwd_f16_f32w(ln, fused, a, vec, cus, P, colsum, dg, db, s);
    }
}

// Byte range [lo, hi) touched by an [N, H] tensor with row stride ld.
struct Span {
    uintptr_t lo = 0, hi = 0;
    bool empty() const { return hi <= lo; }
};

Span span2d(const void *p, int64_t N, int64_t H, int64_t ld, size_t e) {
    Span s;
    if (!p || N <= 0 || H <= 0) return s;
    s.lo = (uintptr_t)p;
    s.hi = s.lo + (size_t)((N - 1) * ld + H) * e;
    return s;
}
Span span1d(const void *p, int64_t n, size_t e) { return span2d(p, 1, n, n, e); }

bool overlaps(const Span &a, const Span &b) {
    if (a.empty() || b.empty()) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Sizes: H in [1, max], N >= 0, strides >= H, and the addressed extent must
// stay far from int64 overflow.
int check_shape(int64_t N, int64_t H) {
    if (N < 0 || H <= 0) return RN_EINVAL;
    if (H > kMaxHidden) return RN_EUNSUPPORTED;
    return RN_OK;
}
int check_ld(int64_t ld, int64_t N, int64_t H) {
    if (ld < H) return RN_EINVAL;
    // (N-1)*ld + H elements must fit comfortably in 2^60 bytes
    if (N > 0 && ld > ((int64_t)1 << 58) / (N > 0 ? N : 1)) return RN_EINVAL;
    return RN_OK;
}
// eps must be a finite, positive, normal float (the kernels' reciprocal
// square root of var + eps is then always taken of a normal number).
int check_eps(float eps) {
    if (!(eps >= FLT_MIN) || !isfinite(eps)) return RN_EINVAL;
    return RN_OK;
}

// The 16-byte vector path needs H, every row stride and every row/vector
// base address to be multiples of 16 bytes.
struct VecCheck {
    size_t e;
    int64_t H;
    bool ok;
    VecCheck(size_t e_, int64_t H_) : e(e_), H(H_), ok((H_ * (int64_t)e_) % 16 == 0) {}
    void ptr(const void *p) { if (p && !aligned(p, 16)) ok = false; }
    void ld(int64_t l) { if ((l * (int64_t)e) % 16 != 0) ok = false; }
};

int hip_status(hipError_t e) { return e == hipSuccess ? RN_OK : RN_EHIP; }

}  // namespace

#define RN_TRY(expr)                 \
    do {                             \
        int rn_st_ = (expr);         \
        if (rn_st_ != RN_OK) return rn_st_; \
    } while (0)

// ------------------------------------------------------------------ forward --
static int fwd_common(int op, const void *x, int64_t ldx, const void *res,
                      int64_t ldr, const void *gamma, const void *beta, void *y,
                      int64_t ldy, void *h, int64_t ldh, float *mean,
                      float *rstd, int64_t N, int64_t H, int dtype, float eps,
                      hipStream_t stream) {
    if (!dtype_ok(dtype)) return RN_EDTYPE;
    RN_TRY(check_shape(N, H));
    RN_TRY(check_eps(eps));
    const size_t e = elem_size(dtype), ep = param_size(dtype);
    // Row tensors may be NULL only when there are no rows.
    if (!gamma || (N > 0 && (!x || !y))) return RN_EINVAL;
    if (op == OP_FUSED && N > 0 && (!res || !h)) return RN_EINVAL;
    RN_TRY(check_ld(ldx, N, H));
    RN_TRY(check_ld(ldy, N, H));
    if (op == OP_FUSED) {
        RN_TRY(check_ld(ldr, N, H));
        RN_TRY(check_ld(ldh, N, H));
    }
    const void *ptrs[] = {x, res, gamma, beta, y, h};
    for (const void *p : std::initializer_list<const void *>{x, res, y, h})
        if (p && !aligned(p, e)) return RN_EINVAL;
    for (const void *p : std::initializer_list<const void *>{gamma, beta})
        if (p && !aligned(p, ep)) return RN_EINVAL;
    if ((mean && !aligned(mean, 4)) || (rstd && !aligned(rstd, 4)))
        return RN_EINVAL;

    // Overlaps.  Inputs: x, res, gamma, beta.  Outputs: y, h, mean, rstd.
    // h may be exactly x or exactly res (in-place residual update).
    const Span sx = span2d(x, N, H, ldx, e), sr = span2d(res, N, H, ldr, e);
    const Span sg = span1d(gamma, H, ep), sb = span1d(beta, H, ep);
    const Span sy = span2d(y, N, H, ldy, e), sh = span2d(h, N, H, ldh, e);
    const Span sm = span1d(mean, N, 4), ss = span1d(rstd, N, 4);
    const Span ins[] = {sx, sr, sg, sb};
    const Span outs[] = {sy, sh, sm, ss};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j) {
            if (i == 1 && ((j == 0 && h == x && ldh == ldx) ||
                           (j == 1 && h == res && ldh == ldr)))
                continue;   // the documented in-place forms
            if (overlaps(outs[i], ins[j])) return RN_EOVERLAP;
        }
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return RN_EOVERLAP;
    }
    if (op == OP_FUSED && h == x && h == res) return RN_EOVERLAP;

    VecCheck vc(e, H);
    for (const void *p : ptrs) vc.ptr(p);
    vc.ld(ldx);
    vc.ld(ldy);
    if (op == OP_FUSED) {
        vc.ld(ldr);
        vc.ld(ldh);
    }

    if (N == 0) return RN_OK;
    int cus = 0;
    RN_TRY(current_cus(&cus));

    FwdArgs a{};
    a.x = x; a.res = res; a.gamma = gamma; a.beta = beta;
    a.y = y; a.h = h; a.mean = mean; a.rstd = rstd;
    a.ldx = ldx; a.ldr = ldr; a.ldy = ldy; a.ldh = ldh;
    a.N = N; a.H = (int)H; a.eps = eps; a.inv_H = 1.0f / (float)H;
    return hip_status(launch_fwd(dtype, op, a, vc.ok, cus, stream));
}

extern "C" int ln_fwd(const void *x, int64_t ldx, const void *gamma,
                      const void *beta, void *y, int64_t ldy, float *mean,
                      float *rstd, int64_t N, int64_t H, int dtype, float eps,
                      hipStream_t stream) {
    return fwd_common(OP_LN, x, ldx, nullptr, 0, gamma, beta, y, ldy, nullptr,
                      0, mean, rstd, N, H, dtype, eps, stream);
}

extern "C" int rms_fwd(const void *x, int64_t ldx, const void *gamma, void *y,
                       int64_t ldy, float *rstd, int64_t N, int64_t H,
                       int dtype, float eps, hipStream_t stream) {
    return fwd_common(OP_RMS, x, ldx, nullptr, 0, gamma, nullptr, y, ldy,
                      nullptr, 0, nullptr, rstd, N, H, dtype, eps, stream);
}

extern "C" int fused_add_rms_fwd(const void *x, int64_t ldx,
                                 const void *residual, int64_t ldr,
                                 const void *gamma, void *y, int64_t ldy,
                                 void *h, int64_t ldh, float *rstd, int64_t N,
                                 int64_t H, int dtype, float eps,
                                 hipStream_t stream) {
    return fwd_common(OP_FUSED, x, ldx, residual, ldr, gamma, nullptr, y, ldy,
                      h, ldh, nullptr, rstd, N, H, dtype, eps, stream);
}

// ----------------------------------------------------------------- backward --
static bool bwd_vec_ok(size_t e, int64_t H, const void *const *ptrs, int np,
                       const int64_t *lds, int nl) {
    VecCheck vc(e, H);
    for (int i = 0; i < np; ++i) vc.ptr(ptrs[i]);
    for (int i = 0; i < nl; ++i) vc.ld(lds[i]);
    return vc.ok;
}

static int partial_rows(int dtype, int64_t N, int64_t H, bool vec, int cus) {
    return bwd_partials(dtype, N, (int)H, vec, cus);
}

static int workspace_bytes_here(int64_t N, int64_t H, int dtype, int is_layernorm,
                                size_t *bytes) {
    int cus = 0;
    RN_TRY(current_cus(&cus));
    // The vector and element-wise plans may differ; size for the larger of
    // the two that use partial rows (the column-sum strategy needs none).
    const int e = (int)elem_size(dtype);
    size_t need = 0;
    bool any = false;
    for (int v = 0; v < 2; ++v) {
        const int P = partial_rows(dtype, N, H, v == 0, cus);
        if (P < 0) continue;
        any = true;
        if (bwd_force_colsum(H, v == 0) ||
            bwd_use_colsum(N, (int)H, e, P, is_layernorm != 0, cus))
            continue;
        // one workgroup of a register plan writes dgamma/dbeta itself
        if (P == 1 && !is_long_row(H, v == 0)) continue;
        const size_t b = (size_t)partial_stride(P) * (size_t)H * sizeof(float) *
                         (is_layernorm ? 2 : 1);
        if (b > need) need = b;
    }
    if (!any) return RN_EUNSUPPORTED;
    *bytes = need;
    return RN_OK;
}

extern "C" int rn_bwd_partial_rows(int64_t N, int64_t H, int dtype, int is_layernorm,
                                   int vectorizable, int *rows) {
    if (!rows) return RN_EINVAL;
    if (!dtype_ok(dtype)) return RN_EDTYPE;
    RN_TRY(check_shape(N, H));
    if (N == 0) {
        *rows = 0;
        return RN_OK;
    }
    int cus = 0;
    RN_TRY(current_cus(&cus));
    const bool vec = vectorizable != 0;
    const int P = partial_rows(dtype, N, H, vec, cus);
    if (P < 0) return RN_EUNSUPPORTED;
    // the same choice as the backward entry points make
    const bool colsum = bwd_force_colsum(H, vec) ||
                        bwd_use_colsum(N, (int)H, (int)elem_size(dtype), P,
                                       is_layernorm != 0, cus);
    *rows = (colsum || (P == 1 && !is_long_row(H, vec))) ? 0 : P;
    return RN_OK;
}

extern "C" int rn_bwd_workspace_bytes(int64_t N, int64_t H, int dtype,
                                      int is_layernorm, int device, size_t *bytes) {
    if (!bytes || device < -1) return RN_EINVAL;
    if (!dtype_ok(dtype)) return RN_EDTYPE;
    RN_TRY(check_shape(N, H));
    if (N == 0) {
        *bytes = 0;
        return RN_OK;
    }
    if (device == -1) return workspace_bytes_here(N, H, dtype, is_layernorm, bytes);
    // another device: make it current for the query, then restore
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return RN_EHIP;
    if (device != cur && hipSetDevice(device) != hipSuccess) return RN_EHIP;
    const int st = workspace_bytes_here(N, H, dtype, is_layernorm, bytes);
    if (device != cur && hipSetDevice(cur) != hipSuccess) return RN_EHIP;
    return st;
}

// Shared by the three backward entry points.  `fused` = the fused
// add+RMSNorm backward: `add` (may be NULL) is added to dx, `dx2` (may be
// NULL) receives a copy of dx; dx may be exactly `add` (in-place
// accumulation of the residual-stream gradient).
static int bwd_common(bool ln, bool fused, const void *dy, int64_t lddy,
                      const void *x, int64_t ldx, const void *gamma,
                      const float *mean, const float *rstd, const void *add,
                      int64_t ldadd, void *dx, int64_t lddx, void *dx2,
                      int64_t lddx2, void *dgamma, void *dbeta, void *workspace,
                      size_t workspace_bytes, int64_t N, int64_t H, int dtype,
                      float eps, hipStream_t stream) {
    if (!dtype_ok(dtype)) return RN_EDTYPE;
    RN_TRY(check_shape(N, H));
    RN_TRY(check_eps(eps));
    const size_t e = elem_size(dtype), ep = param_size(dtype);
    // Row tensors and saved statistics may be NULL only when there are no
    // rows; the parameter gradients are always written.
    if (!gamma || !dgamma || (ln && !dbeta)) return RN_EINVAL;
    if (N > 0 && (!dy || !x || !rstd || !dx || (ln && !mean))) return RN_EINVAL;
    RN_TRY(check_ld(lddy, N, H));
    RN_TRY(check_ld(ldx, N, H));
    RN_TRY(check_ld(lddx, N, H));
    if (fused && add) RN_TRY(check_ld(ldadd, N, H));
    if (fused && dx2) RN_TRY(check_ld(lddx2, N, H));
    if (!fused) {
        add = nullptr;
        dx2 = nullptr;
    }
    const void *ptrs[] = {dy, x, gamma, dx, dgamma, ln ? dbeta : nullptr, add, dx2};
    for (const void *p : std::initializer_list<const void *>{dy, x, dx, add, dx2})
        if (p && !aligned(p, e)) return RN_EINVAL;
    for (const void *p : std::initializer_list<const void *>{gamma, dgamma, ln ? dbeta : nullptr})
        if (p && !aligned(p, ep)) return RN_EINVAL;
    if ((rstd && !aligned(rstd, 4)) || (mean && !aligned(mean, 4))) return RN_EINVAL;
    if (workspace && !aligned(workspace, 256)) return RN_EINVAL;

    const Span sdy = span2d(dy, N, H, lddy, e), sx = span2d(x, N, H, ldx, e);
    const Span sg = span1d(gamma, H, ep);
    const Span sm = span1d(ln ? mean : nullptr, N, 4), ss = span1d(rstd, N, 4);
    const Span sa = span2d(add, N, H, ldadd, e);
    const Span sdx = span2d(dx, N, H, lddx, e), sdx2 = span2d(dx2, N, H, lddx2, e);
    const Span sdg = span1d(dgamma, H, ep), sdb = span1d(ln ? dbeta : nullptr, H, ep);
    const Span sw = span1d(workspace, (int64_t)workspace_bytes, 1);
    const Span ins[] = {sdy, sx, sg, sm, ss, sa};
    const Span outs[] = {sdx, sdx2, sdg, sdb, sw};
    const bool dx_is_add = add && dx == add && lddx == ldadd;
    for (int i = 0; i < 5; ++i) {
        for (int j = 0; j < 6; ++j) {
            if (i == 0 && j == 5 && dx_is_add) continue;   // in-place accumulate
            if (overlaps(outs[i], ins[j])) return RN_EOVERLAP;
        }
        for (int j = i + 1; j < 5; ++j)
            if (overlaps(outs[i], outs[j])) return RN_EOVERLAP;
    }

    const int64_t lds[] = {lddy, ldx, lddx, add ? ldadd : lddx, dx2 ? lddx2 : lddx};
    const bool vec = bwd_vec_ok(e, H, ptrs, 8, lds, 5);
    int cus = 0;
    RN_TRY(current_cus(&cus));
    const int P = N == 0 ? 0 : partial_rows(dtype, N, H, vec, cus);
    if (P < 0) return RN_EUNSUPPORTED;
    const bool colsum =
        N > 0 && (bwd_force_colsum(H, vec) || bwd_use_colsum(N, (int)H, (int)e, P, ln, cus));
    // no partial rows: the column sums, or one workgroup of a register plan
    // (kernel 1 then writes dgamma/dbeta itself)
    const bool no_partials = colsum || (P == 1 && !is_long_row(H, vec));
    const size_t need = no_partials ? 0
                                    : (size_t)partial_stride(P) * (size_t)H * sizeof(float) *
                                          (ln ? 2 : 1);
    if (need > 0 && (!workspace || workspace_bytes < need)) return RN_EWORKSPACE;

    BwdArgs a{};
    a.dy = dy; a.x = x; a.gamma = gamma; a.mean = mean; a.rstd = rstd;
    a.dx = dx; a.part = (float *)workspace; a.add = add; a.dx2 = dx2;
    a.dgamma = dgamma; a.dbeta = dbeta;
    a.lddy = lddy; a.ldx = ldx; a.lddx = lddx; a.ldadd = ldadd; a.lddx2 = lddx2;
    a.N = N; a.H = (int)H; a.inv_H = 1.0f / (float)H;
    return hip_status(
        launch_bwd(dtype, ln, fused, a, vec, cus, P, colsum, dgamma, dbeta, stream));
}

extern "C" int ln_bwd(const void *dy, int64_t lddy, const void *x, int64_t ldx,
                      const void *gamma, const float *mean, const float *rstd,
                      void *dx, int64_t lddx, void *dgamma, void *dbeta,
                      void *workspace, size_t workspace_bytes, int64_t N,
                      int64_t H, int dtype, float eps, hipStream_t stream) {
    return bwd_common(true, false, dy, lddy, x, ldx, gamma, mean, rstd, nullptr, 0,
                      dx, lddx, nullptr, 0, dgamma, dbeta, workspace,
                      workspace_bytes, N, H, dtype, eps, stream);
}

// ------------------------------------------------ no-allocation backward --
// ln_bwd_noalloc keeps its partial rows in this array instead of a caller
// workspace: one copy per GPU the library runs on, held until the process
// ends.  On the host the array's name is only a stand-in for the symbol,
// not a device address: host code uses the address hipGetSymbolAddress
// returns for the current device (scratch_here), never the name.  Kernel 1
// writes every partial-row slot kernel 2 reads, within the same call, so
// nothing in it has to start at zero; calls on one GPU share it, and calls
// whose work overlaps in time on that GPU (two streams) race.
static __device__ __align__(256) unsigned char scratch[RN_NOALLOC_MAX_WORKSPACE_BYTES];

namespace {
void *g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) on the first call there.
int scratch_here(void **p) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return RN_EHIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *q = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? q : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return RN_EHIP;
    *p = g_scratch[dev];
    return RN_OK;
}
}  // namespace

extern "C" int ln_bwd_noalloc(const void *dy, int64_t lddy, const void *x,
                              int64_t ldx, const void *gamma, const float *mean,
                              const float *rstd, void *dx, int64_t lddx,
                              void *dgamma, void *dbeta, int64_t N, int64_t H,
                              int dtype, float eps, hipStream_t stream) {
    void *ws = nullptr;
    RN_TRY(scratch_here(&ws));
    // the same checks and kernels as ln_bwd; a shape whose partial rows
    // exceed the array is RN_EWORKSPACE before anything is enqueued
    return bwd_common(true, false, dy, lddy, x, ldx, gamma, mean, rstd, nullptr, 0,
                      dx, lddx, nullptr, 0, dgamma, dbeta, ws,
                      RN_NOALLOC_MAX_WORKSPACE_BYTES, N, H, dtype, eps, stream);
}

extern "C" int rms_bwd(const void *dy, int64_t lddy, const void *x,
                       int64_t ldx, const void *gamma, const float *rstd,
                       void *dx, int64_t lddx, void *dgamma, void *workspace,
                       size_t workspace_bytes, int64_t N, int64_t H, int dtype,
                       float eps, hipStream_t stream) {
    return bwd_common(false, false, dy, lddy, x, ldx, gamma, nullptr, rstd, nullptr,
                      0, dx, lddx, nullptr, 0, dgamma, nullptr, workspace,
                      workspace_bytes, N, H, dtype, eps, stream);
}

extern "C" int fused_add_rms_bwd(const void *dy, int64_t lddy, const void *h,
                                 int64_t ldh, const void *gamma, const float *rstd,
                                 const void *dh_in, int64_t lddh_in, void *dx,
                                 int64_t lddx, void *dres, int64_t lddres,
                                 void *dgamma, void *workspace,
                                 size_t workspace_bytes, int64_t N, int64_t H,
                                 int dtype, float eps, hipStream_t stream) {
    return bwd_common(false, true, dy, lddy, h, ldh, gamma, nullptr, rstd, dh_in,
                      lddh_in, dx, lddx, dres, lddres, dgamma, nullptr, workspace,
                      workspace_bytes, N, H, dtype, eps, stream);
}

// ------------------------------------------------------------------- misc --
extern "C" int64_t rn_max_hidden(int dtype, int vectorizable) {
    if (!dtype_ok(dtype)) return 0;
    (void)vectorizable;   // both paths walk long rows in segments
    return kMaxHidden;
}

extern "C" const char *rn_status_str(int status) {
    switch (status) {
    case RN_OK: return "ok";
    case RN_EINVAL: return "invalid argument (size, stride, eps, NULL or misaligned pointer)";
    case RN_EDTYPE: return "unknown dtype";
    case RN_EOVERLAP: return "an output overlaps an input or another output";
    case RN_EWORKSPACE: return "backward workspace missing or too small";
    case RN_EHIP: return "HIP runtime error";
    case RN_EUNSUPPORTED: return "row length above the supported maximum";
    default: return "unknown status";
    }
}

extern "C" int rn_copy(const void *src, void *dst, size_t bytes,
                       hipStream_t stream) {
    if (bytes == 0) return RN_OK;
    if (!src || !dst) return RN_EINVAL;
    const Span a = span1d(src, (int64_t)bytes, 1), b = span1d(dst, (int64_t)bytes, 1);
    if (overlaps(a, b)) return RN_EOVERLAP;
    return hip_status(launch_copy(src, dst, bytes, stream));
}

extern "C" int rn_add(const void *a, const void *b, void *out, int64_t n, int dtype,
                      hipStream_t stream) {
    if (!dtype_ok(dtype)) return RN_EDTYPE;
    if (n < 0) return RN_EINVAL;
    if (n == 0) return RN_OK;
    if (!a || !b || !out) return RN_EINVAL;
    const size_t e = elem_size(dtype);
    for (const void *p : {a, b, (const void *)out})
        if (!aligned(p, e)) return RN_EINVAL;
    const Span sa = span1d(a, n, e), sb = span1d(b, n, e), so = span1d(out, n, e);
    if ((out != a && overlaps(so, sa)) || (out != b && overlaps(so, sb)))
        return RN_EOVERLAP;
    const int elem = dtype == RN_F32 ? 0 : (dtype == RN_BF16 || dtype == RN_BF16_F32W) ? 1 : 2;
    return hip_status(launch_add(elem, a, b, out, n, stream));
}
