/*
 * rownorm.h - row-wise LayerNorm / RMSNorm / fused residual-add + RMSNorm,
 * forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI of librownorm.so.  Every tensor argument is a DEVICE pointer
 * owned by the caller; the library allocates nothing, keeps no buffers, and
 * never synchronizes.  Every compute entry point only validates its
 * arguments and enqueues kernels on `stream` (0 = the null stream of the
 * current device), then returns.  The current HIP device must be the device
 * that owns the pointers and the stream.
 *
 * Shapes.  A tensor argument "[N, H]" is N rows of H elements, row-major,
 * with a row stride ld (in ELEMENTS, ld >= H) and contiguous elements within
 * a row.  Normalization is over the last dimension (the H elements of one
 * row); rows are independent.  Callers with (B, T, H) inputs pass N = B*T.
 * gamma, beta, dgamma, dbeta are vectors of H elements shared by all rows
 * (no row offset is ever applied to them).
 *
 * Types.  One `dtype` (rn_dtype) names the storage of every tensor of a
 * call: the activations (x, residual, h, y, dy, dx, dh_in, dres) and the
 * parameters (gamma, beta, dgamma, dbeta), which are either of the
 * activation type or, with the *_F32W codes, float32 ("Write Cuda Layernorm
 * Kernel", Required reasoning process and Kernel design rules, keep the
 * affine parameters in float32 whatever the activations are).  mean and
 * rstd are always float32 vectors of N elements.  All arithmetic runs in
 * float32 after the load; results are rounded to their storage type (round
 * to nearest even; fp16 overflow gives infinity) at the store.
 *
 * eps.  Added INSIDE the square root: rstd = 1 / sqrt(var + eps).  It must be
 * a finite, positive, normal float (>= FLT_MIN, about 1.2e-38); anything
 * else is RN_EINVAL.  rstd comes from the hardware reciprocal square root
 * (within about 1 ulp of the exact value).
 *
 * Status.  Every function returns RN_OK (0) or a negative RN_E* code.  All
 * argument checks run before anything is enqueued: a non-zero return means
 * nothing was launched.  RN_EHIP means a HIP call failed after the checks
 * (e.g. the launch itself); rn_status_str() names every code.
 *
 * Pages these operations follow (cited by title and section):
 *  "Write Triton Layernorm Kernel": Required reasoning process (row per
 *      program, mean over H, variance, rstd with eps inside the root,
 *      affine, saved mean/rstd); Kernel design rules; Correctness
 *      requirements.
 *  "Write Cuda Layernorm Kernel": Required reasoning process (two-pass and
 *      Welford statistics, the parallel merge, RMSNorm, the backward
 *      formulas); Kernel design rules.
 *  "Write Triton Fused Add Rmsnorm Kernel": Required reasoning process
 *      (fp32 add, write-back of h in the same pass, RMSNorm of h, in-place
 *      aliasing rules); Correctness requirements.
 *  "Rewrite Triton normalization backward kernel_1 (#499)": Summary
 *      (per-row grad_input, parameter gradients through a bounded set of
 *      fp32 partial rows reduced by a second kernel, program count a small
 *      multiple of the compute-unit count).
 */
#ifndef ROWNORM_H
#define ROWNORM_H

#include <stddef.h>
#include <stdint.h>
/* hipStream_t.  hipcc defines __HIP_PLATFORM_AMD__ itself; a plain C or C++
 * compiler needs -D__HIP_PLATFORM_AMD__ and the ROCm include directory, and
 * links with -lrownorm. */
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RN_F32 = 0,         /* float32 activations and parameters               */
    RN_BF16 = 1,        /* bfloat16 activations and parameters              */
    RN_F16 = 2,         /* IEEE binary16 activations and parameters         */
    RN_BF16_F32W = 3,   /* bfloat16 activations, float32 parameters         */
    RN_F16_F32W = 4     /* binary16 activations, float32 parameters         */
} rn_dtype;

enum {
    RN_OK = 0,
    RN_EINVAL = -1,        /* bad size, stride, eps, NULL or misaligned ptr */
    RN_EDTYPE = -2,        /* unknown dtype                                 */
    RN_EOVERLAP = -3,      /* an output overlaps an input or another output */
    RN_EWORKSPACE = -4,    /* backward workspace missing or too small       */
    RN_EHIP = -5,          /* a HIP runtime call failed                     */
    RN_EUNSUPPORTED = -6   /* H above the longest row (rn_max_hidden)         */
};

/* LayerNorm forward ("Write Triton Layernorm Kernel", Required reasoning
 * process, steps 1-10; "Write Cuda Layernorm Kernel", steps 2, 5, 6, 7).
 * Per row:  mean = sum(x)/H,  var = sum((x - mean)^2)/H,
 *           rstd = 1/sqrt(var + eps),
 *           y = (x - mean) * rstd * gamma + beta.
 *   x     [N, H] in, row stride ldx          gamma [H] in
 *   beta  [H] in, or NULL for no bias        y     [N, H] out, stride ldy
 *   mean, rstd  [N] float32 out, each may be NULL (not written)
 * y may not overlap any input; mean/rstd may not overlap anything. */
int ln_fwd(const void *x, int64_t ldx, const void *gamma, const void *beta,
           void *y, int64_t ldy, float *mean, float *rstd,
           int64_t N, int64_t H, int dtype, float eps, hipStream_t stream);

/* RMSNorm forward ("Write Cuda Layernorm Kernel", Required reasoning
 * process, step 5 and Kernel design rules).  No mean subtraction, no bias:
 *   rstd = 1/sqrt(sum(x^2)/H + eps),  y = x * rstd * gamma.
 *   x [N, H] in; gamma [H] in; y [N, H] out; rstd [N] float32 out or NULL. */
int rms_fwd(const void *x, int64_t ldx, const void *gamma, void *y,
            int64_t ldy, float *rstd, int64_t N, int64_t H, int dtype,
            float eps, hipStream_t stream);

/* Fused residual add + RMSNorm forward ("Write Triton Fused Add Rmsnorm
 * Kernel", Required reasoning process, steps 1-9):
 *   h = x + residual (in float32), stored rounded to dtype in the same pass;
 *   y = h * rstd * gamma with rstd = 1/sqrt(sum(h^2)/H + eps), computed from
 *   the UNROUNDED float32 h.
 *   x, residual [N, H] in (strides ldx, ldr); gamma [H] in;
 *   y [N, H] out (ldy); h [N, H] out (ldh); rstd [N] float32 out or NULL.
 * In-place residual update is allowed: h may be EXACTLY x (same pointer and
 * ldh == ldx) or exactly residual; each element is read before it is
 * written.  Any other overlap is RN_EOVERLAP. */
int fused_add_rms_fwd(const void *x, int64_t ldx, const void *residual,
                      int64_t ldr, const void *gamma, void *y, int64_t ldy,
                      void *h, int64_t ldh, float *rstd, int64_t N, int64_t H,
                      int dtype, float eps, hipStream_t stream);

/* LayerNorm backward ("Write Cuda Layernorm Kernel", Required reasoning
 * process, step 8; "Rewrite Triton normalization backward kernel_1 (#499)",
 * Summary).  With x_hat = (x - mean) * rstd and g = dy * gamma, per row:
 *   c1 = sum(g)/H,  c2 = sum(g * x_hat)/H,
 *   dx = rstd * (g - c1 - x_hat * c2);
 * and over all rows: dgamma = sum(dy * x_hat), dbeta = sum(dy).
 *   dy, x  [N, H] in;  gamma [H] in;
 *   mean, rstd [N] float32 in: the statistics saved by ln_fwd (required;
 *     eps is already inside rstd, so `eps` is only validated);
 *   dx [N, H] out;  dgamma, dbeta [H] out (required);
 *   workspace: device scratch of at least rn_bwd_workspace_bytes(N, H,
 *     dtype, 1, device) bytes, 256-byte aligned, owned by the caller; it holds the
 *     float32 partial rows between the two kernels and must not be touched
 *     until the call's work on `stream` is done.  NULL is fine when that size
 *     is 0.
 * The partial-row count is fixed by (N, H, dtype, device), so results are
 * bitwise reproducible run to run.  N = 0 writes dgamma = dbeta = 0. */
int ln_bwd(const void *dy, int64_t lddy, const void *x, int64_t ldx,
           const void *gamma, const float *mean, const float *rstd, void *dx,
           int64_t lddx, void *dgamma, void *dbeta, void *workspace,
           size_t workspace_bytes, int64_t N, int64_t H, int dtype, float eps,
           hipStream_t stream);

/* ln_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture that may not call hipMalloc,
 * tight serving loops, harnesses that forbid allocation).  The partial rows
 * live in a static device array of RN_NOALLOC_MAX_WORKSPACE_BYTES inside
 * the library, one per GPU, held until the process ends; the call itself
 * allocates nothing.  Same arguments, checks, kernels and results (bit for
 * bit) as ln_bwd with a caller workspace.  A shape whose partial rows need
 * more than RN_NOALLOC_MAX_WORKSPACE_BYTES (rn_bwd_workspace_bytes(N, H,
 * dtype, 1, device) larger than it) returns RN_EWORKSPACE and enqueues
 * nothing.  All calls on one GPU share its array: calls whose work may
 * overlap in time on that GPU (e.g. on two streams) race and must be
 * ordered by the caller.  The first call on each GPU looks up the array's
 * address there (RN_EHIP if that fails); make it outside graph capture. */
#define RN_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)32 << 20)
int ln_bwd_noalloc(const void *dy, int64_t lddy, const void *x, int64_t ldx,
                   const void *gamma, const float *mean, const float *rstd,
                   void *dx, int64_t lddx, void *dgamma, void *dbeta, int64_t N,
                   int64_t H, int dtype, float eps, hipStream_t stream);

/* RMSNorm backward.  The pages ask for it but print no formula; it is the
 * derivative of rms_fwd: with x_hat = x * rstd and g = dy * gamma,
 *   c2 = sum(g * x_hat)/H,   dx = rstd * (g - x_hat * c2),
 *   dgamma = sum over rows of dy * x_hat.
 * Arguments as in ln_bwd (no mean, no dbeta). */
int rms_bwd(const void *dy, int64_t lddy, const void *x, int64_t ldx,
            const void *gamma, const float *rstd, void *dx, int64_t lddx,
            void *dgamma, void *workspace, size_t workspace_bytes, int64_t N,
            int64_t H, int dtype, float eps, hipStream_t stream);

/* Fused residual add + RMSNorm backward ("Write Triton Fused Add Rmsnorm
 * Kernel", Required reasoning process, step 10).  The forward computed
 * h = x + residual and y = RMSNorm(h); both inputs get the same gradient
 * dL/dh, which is the RMSNorm backward of the STORED h plus dh_in, the
 * gradient arriving at h through the residual stream (h is also the next
 * block's residual):
 *   dx = dres = rstd * (g - x_hat * c2) + dh_in,  x_hat = h * rstd,
 *   dgamma = sum over rows of dy * x_hat.
 *   dy, h  [N, H] in;  gamma [H] in;  rstd [N] float32 in (from
 *     fused_add_rms_fwd; required);
 *   dh_in [N, H] in, or NULL for no residual-stream gradient;
 *   dx [N, H] out;  dres [N, H] out, or NULL to write the gradient once
 *     (dx then serves both inputs);  dgamma [H] out;
 *   workspace as for rms_bwd (rn_bwd_workspace_bytes(N, H, dtype, 0,
 *     device)).
 * dx may be exactly dh_in (same pointer and stride: in-place accumulation);
 * any other overlap is RN_EOVERLAP. */
int fused_add_rms_bwd(const void *dy, int64_t lddy, const void *h, int64_t ldh,
                      const void *gamma, const float *rstd, const void *dh_in,
                      int64_t lddh_in, void *dx, int64_t lddx, void *dres,
                      int64_t lddres, void *dgamma, void *workspace,
                      size_t workspace_bytes, int64_t N, int64_t H, int dtype,
                      float eps, hipStream_t stream);

/* Bytes of backward workspace ln_bwd / rms_bwd / fused_add_rms_bwd need for
 * (N, H, dtype, LayerNorm or RMSNorm) on GPU `device` (-1: the current
 * device).  The workspace holds the float32 partial rows of dgamma (and
 * dbeta) between the two backward kernels; their count is the first
 * kernel's workgroup count, a small multiple of the compute-unit count, so
 * the size grows with H and with N only up to that count ("Rewrite Triton
 * normalization backward kernel_1 (#499)", Summary: bounded partial rows,
 * program count tied to the CU count).  It depends on dtype because each
 * storage pair has its own team plans, and on the device's CU count.  It
 * is 0 when no partial rows are needed: one workgroup holds every row, or
 * the rows are so few for their width that the backward forms dgamma/dbeta
 * from x and dy directly.
 * Returns RN_OK and sets *bytes (0 for N = 0, without touching any GPU), or
 * RN_EINVAL (bytes NULL, device < -1, bad N/H), RN_EDTYPE, RN_EUNSUPPORTED,
 * or RN_EHIP (the device cannot be queried). */
int rn_bwd_workspace_bytes(int64_t N, int64_t H, int dtype, int is_layernorm,
                           int device, size_t *bytes);

/* Longest row (H) supported for `dtype`: 4194304 elements on both the 16-byte
 * path (rows whose size, stride and base addresses are multiples of 16
 * bytes) and the element-wise path (`vectorizable` = 0).  Rows of up to
 * 16384 (16-byte path; 32768 in the forward of 2-byte rows with 2-byte
 * parameters) or 8192 (element-wise) elements are held in the registers of
 * the register plans; longer rows are walked in segments by one
 * 1024-thread workgroup that keeps as much of the row as fits on chip
 * (first in registers, then in LDS: 160 KiB on MI355X) between the
 * statistics and the output pass and reads the rest twice ("Write Triton
 * Layernorm Kernel", Required reasoning process, large-H loop over column
 * blocks).  The forward holds LayerNorm/RMSNorm bf16 rows of up to 139264
 * elements, fused rows of up to 65536.  Returns 0 for an unknown dtype. */
int64_t rn_max_hidden(int dtype, int vectorizable);

/* Text for a status code.  The argument checks behind the codes follow the
 * pages' launcher duties ("Write Triton Fused Add Rmsnorm Kernel", Required
 * reasoning process: validate shapes, strides and aliasing before launch;
 * "Write Triton Layernorm Kernel", Correctness requirements: reject a
 * non-positive eps).  Never NULL; unknown codes give "unknown status". */
const char *rn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_H */
