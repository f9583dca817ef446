/*
 * Row-wise normalization oracle: a plain, slow, obviously correct CPU
 * definition of what the GPU path computes, in binary64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * never calls it, and it shares no code, header, table or helper with the
 * HIP kernels under rmsnorm_row_welford_amd/csrc.
 *
 * Sources (cited by page title and section):
 *  [LNT]  "Write Triton Layernorm Kernel": Required reasoning process,
 *         steps 1-10; Correctness requirements.
 *  [LNC]  "Write Cuda Layernorm Kernel": Required reasoning process,
 *         step 2 (two-pass and Welford recurrence), step 3 (parallel merge),
 *         step 5 (rstd, RMSNorm), step 8 (backward formulas).
 *  [FAR]  "Write Triton Fused Add Rmsnorm Kernel": Required reasoning
 *         process, steps 3-7 and 10.
 *  [BWD]  "Rewrite Triton normalization backward kernel_1 (#499)": Summary
 *         (parameter gradients are sums over all rows).
 *
 * Conventions fixed here (each one a reading of the pages):
 *  - every reduction divides by the full row length H;
 *  - variance is the population variance, computed two-pass: mean first,
 *    then the sum of squared deviations from it;
 *  - eps is added inside the square root: rstd = 1/sqrt(var + eps);
 *  - RMSNorm has no mean subtraction and no bias;
 *  - the backward recomputes mean/rstd from x in binary64 (it does not read
 *    any saved statistics);
 *  - sums run sequentially in index order.  Rows are independent, so the
 *    row loop may run on several threads without changing any result; the
 *    column sums for dgamma/dbeta run over rows in row order per column.
 *
 * All array arguments are row-major with an explicit row stride ("ld", in
 * elements).  Outputs are binary64; rounding to the storage type is done
 * by the codec functions at the bottom, which are this file's own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Row statistics                                                       */
/* ------------------------------------------------------------------ */

/* Two-pass mean and population variance of one row ([LNC] step 2, first
 * option; [LNT] steps 3 and 5): mean = sum(x)/H, var = sum((x-mean)^2)/H. */
static void row_mean_var(const double *x, int64_t H, double *mean, double *var)
{
    double s = 0.0;
    for (int64_t j = 0; j < H; ++j) s += x[j];
    double mu = s / (double)H;
    double q = 0.0;
    for (int64_t j = 0; j < H; ++j) {
        double d = x[j] - mu;
        q += d * d;
    }
    *mean = mu;
    *var = q / (double)H;
}

/* Mean of squares of one row (the RMSNorm statistic, [LNC] step 5 and
 * design rules; [FAR] step 5): m2 = sum(x^2)/H. */
static double row_mean_sq(const double *x, int64_t H)
{
    double q = 0.0;
    for (int64_t j = 0; j < H; ++j) q += x[j] * x[j];
    return q / (double)H;
}

/* rstd with eps inside the square root ([LNT] step 6; [LNC] step 7). */
static double rstd_of(double var, double eps) { return 1.0 / sqrt(var + eps); }

/* ------------------------------------------------------------------ */
/* Forward passes                                                       */
/* ------------------------------------------------------------------ */

/* LayerNorm forward ([LNT] steps 3-10; [LNC] steps 5-6):
 *   y = (x - mean) * rstd * gamma + beta    (beta == NULL means beta = 0)
 * mean/rstd (length N) are written when non-NULL. */
void orc_ln_fwd(int64_t N, int64_t H, const double *x, int64_t ldx,
                const double *gamma, const double *beta, double eps,
                double *y, int64_t ldy, double *mean, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *xr = x + r * ldx;
        double *yr = y + r * ldy;
        double mu, var;
        row_mean_var(xr, H, &mu, &var);
        double s = rstd_of(var, eps);
        for (int64_t j = 0; j < H; ++j) {
            double xhat = (xr[j] - mu) * s;
            yr[j] = xhat * gamma[j] + (beta ? beta[j] : 0.0);
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = s;
    }
}

/* RMSNorm forward ([LNC] step 5 and design rules; [LNT] step 5):
 *   y = x * rstd * gamma,  rstd = 1/sqrt(mean(x^2) + eps).  No bias. */
void orc_rms_fwd(int64_t N, int64_t H, const double *x, int64_t ldx,
                 const double *gamma, double eps, double *y, int64_t ldy,
                 double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *xr = x + r * ldx;
        double *yr = y + r * ldy;
        double s = rstd_of(row_mean_sq(xr, H), eps);
        for (int64_t j = 0; j < H; ++j) yr[j] = xr[j] * s * gamma[j];
        if (rstd) rstd[r] = s;
    }
}

/* Fused residual add + RMSNorm forward ([FAR] steps 3-7, 9):
 *   h = x + residual (exact in binary64 for bf16/fp32 inputs),
 *   y = RMSNorm(h) computed on the unrounded h.
 * h is returned unrounded; rounding it to the storage type is the codec's
 * job.  h may not alias x or residual here (the oracle keeps things plain). */
void orc_fused_add_rms_fwd(int64_t N, int64_t H, const double *x, int64_t ldx,
                           const double *res, int64_t ldr, const double *gamma,
                           double eps, double *y, int64_t ldy, double *h,
                           int64_t ldh, double *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *xr = x + r * ldx;
        const double *rr = res + r * ldr;
        double *hr = h + r * ldh;
        double *yr = y + r * ldy;
        for (int64_t j = 0; j < H; ++j) hr[j] = xr[j] + rr[j];
        double s = rstd_of(row_mean_sq(hr, H), eps);
        for (int64_t j = 0; j < H; ++j) yr[j] = hr[j] * s * gamma[j];
        if (rstd) rstd[r] = s;
    }
}

/* ------------------------------------------------------------------ */
/* Backward passes                                                      */
/* ------------------------------------------------------------------ */

/* Column sums over all rows for the parameter gradients ([LNC] step 8:
 * dgamma_j = sum over rows of xhat_ij * dy_ij, dbeta_j = sum over rows of
 * dy_ij; [BWD] Summary).  xhat is rebuilt from x with per-row mean and rstd
 * (mean == NULL means RMSNorm: xhat = x * rstd).  Each column is summed over
 * rows in row order; threads split the columns, so the result does not
 * depend on the thread count. */
static void param_grads(int64_t N, int64_t H, const double *dy, int64_t lddy,
                        const double *x, int64_t ldx, const double *mean,
                        const double *rstd, double *dgamma, double *dbeta)
{
    const int64_t CB = 64; /* column block: only for cache locality */
    int64_t nblk = (H + CB - 1) / CB;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblk; ++b) {
        int64_t j0 = b * CB, j1 = j0 + CB < H ? j0 + CB : H;
        double g[64], be[64];
        for (int64_t j = j0; j < j1; ++j) { g[j - j0] = 0.0; be[j - j0] = 0.0; }
        for (int64_t r = 0; r < N; ++r) {
            const double *xr = x + r * ldx;
            const double *dyr = dy + r * lddy;
            double mu = mean ? mean[r] : 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                double xhat = (xr[j] - mu) * rstd[r];
                g[j - j0] += dyr[j] * xhat;
                be[j - j0] += dyr[j];
            }
        }
        for (int64_t j = j0; j < j1; ++j) {
            dgamma[j] = g[j - j0];
            if (dbeta) dbeta[j] = be[j - j0];
        }
    }
}

/* LayerNorm backward ([LNC] step 8).  With g = dy * gamma (the gradient with
 * respect to xhat), per row:
 *   c1 = sum(g)/H,  c2 = sum(g * xhat)/H,
 *   dx = rstd * (g - c1 - xhat * c2),
 * which is the page's formula with the 1/D factor distributed.
 * dgamma/dbeta are the column sums above.  mean_out/rstd_out (length N,
 * required) receive the binary64 statistics recomputed from x; the column
 * sums read them back. */
void orc_ln_bwd(int64_t N, int64_t H, const double *dy, int64_t lddy,
                const double *x, int64_t ldx, const double *gamma, double eps,
                double *dx, int64_t lddx, double *dgamma, double *dbeta,
                double *mean_out, double *rstd_out)
{
    double *mu = mean_out, *rs = rstd_out;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *xr = x + r * ldx;
        const double *dyr = dy + r * lddy;
        double *dxr = dx + r * lddx;
        double m, var;
        row_mean_var(xr, H, &m, &var);
        double s = rstd_of(var, eps);
        double sg = 0.0, sgx = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double xhat = (xr[j] - m) * s;
            double g = dyr[j] * gamma[j];
            sg += g;
            sgx += g * xhat;
        }
        double c1 = sg / (double)H, c2 = sgx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            double xhat = (xr[j] - m) * s;
            double g = dyr[j] * gamma[j];
            dxr[j] = s * (g - c1 - xhat * c2);
        }
        mu[r] = m;
        rs[r] = s;
    }
    param_grads(N, H, dy, lddy, x, ldx, mu, rs, dgamma, dbeta);
}

/* RMSNorm backward.  The pages state the need for it but print no formula;
 * it follows from differentiating y = x * rstd * gamma with
 * rstd = (mean(x^2) + eps)^(-1/2), whose derivative is
 * d rstd / d x_k = -rstd^3 x_k / H.  With xhat = x * rstd, g = dy * gamma:
 *   c2 = sum(g * xhat)/H,   dx = rstd * (g - xhat * c2),
 *   dgamma = column sums of dy * xhat.
 * rstd_out (required) receives the recomputed binary64 rstd. */
void orc_rms_bwd(int64_t N, int64_t H, const double *dy, int64_t lddy,
                 const double *x, int64_t ldx, const double *gamma, double eps,
                 double *dx, int64_t lddx, double *dgamma, double *rstd_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *xr = x + r * ldx;
        const double *dyr = dy + r * lddy;
        double *dxr = dx + r * lddx;
        double s = rstd_of(row_mean_sq(xr, H), eps);
        double sgx = 0.0;
        for (int64_t j = 0; j < H; ++j) sgx += dyr[j] * gamma[j] * (xr[j] * s);
        double c2 = sgx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            double xhat = xr[j] * s;
            double g = dyr[j] * gamma[j];
            dxr[j] = s * (g - xhat * c2);
        }
        rstd_out[r] = s;
    }
    param_grads(N, H, dy, lddy, x, ldx, NULL, rstd_out, dgamma, NULL);
}

/* Fused residual add + RMSNorm backward ("Write Triton Fused Add Rmsnorm
 * Kernel", Required reasoning process, step 10).  The forward computed
 * h = x + residual and y = RMSNorm(h); since dh/dx = dh/dresidual = 1, both
 * inputs receive the same gradient dL/dh.  It is the RMSNorm backward at the
 * stored h with the rstd the forward saved (the forward took it from the
 * unrounded h; the backward has only the stored h), plus dh_in, the gradient
 * that reaches h through the residual stream (h is also the next block's
 * residual; NULL means none).  With xhat = h * rstd and g = dy * gamma:
 *   c2 = sum(g * xhat)/H,   dx = dres = rstd * (g - xhat * c2) + dh_in,
 *   dgamma = column sums of dy * xhat. */
void orc_fused_add_rms_bwd(int64_t N, int64_t H, const double *dy, int64_t lddy,
                           const double *h, int64_t ldh, const double *gamma,
                           const double *rstd, const double *dh_in, int64_t lddh,
                           double *dx, int64_t lddx, double *dgamma)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        const double *hr = h + r * ldh;
        const double *dyr = dy + r * lddy;
        double *dxr = dx + r * lddx;
        double s = rstd[r];
        double sgx = 0.0;
        for (int64_t j = 0; j < H; ++j) sgx += dyr[j] * gamma[j] * (hr[j] * s);
        double c2 = sgx / (double)H;
        for (int64_t j = 0; j < H; ++j) {
            double g = dyr[j] * gamma[j];
            dxr[j] = s * (g - (hr[j] * s) * c2);
        }
        if (dh_in)
            for (int64_t j = 0; j < H; ++j) dxr[j] += dh_in[r * lddh + j];
    }
    param_grads(N, H, dy, lddy, h, ldh, NULL, rstd, dgamma, NULL);
}

/* ------------------------------------------------------------------ */
/* Welford recurrence and parallel merge (for self-checks only)         */
/* ------------------------------------------------------------------ */

/* Sequential Welford over n values ([LNC] step 2, second option):
 *   count += 1; delta = x - mean; mean += delta/count;
 *   M2 += delta * (x - new mean).
 * Returns (count, mean, M2); the variance is M2 / count. */
void orc_welford(const double *x, int64_t n, double *count, double *mean,
                 double *m2)
{
    double c = 0.0, m = 0.0, q = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        c += 1.0;
        double d_old = x[i] - m;
        m += d_old / c;
        q += d_old * (x[i] - m);
    }
    *count = c;
    *mean = m;
    *m2 = q;
}

/* Parallel merge of two Welford states ([LNC] step 3):
 *   n = na + nb, delta = mb - ma, mean = ma + delta*nb/n,
 *   M2 = M2a + M2b + delta^2 * na*nb/n.
 * A state with count 0 is the identity ([LNC] step 4). */
void orc_welford_merge(double na, double ma, double m2a, double nb, double mb,
                       double m2b, double *n, double *mean, double *m2)
{
    double nn = na + nb;
    if (nn == 0.0) { *n = 0.0; *mean = 0.0; *m2 = 0.0; return; }
    double d = mb - ma;
    *n = nn;
    *mean = ma + d * (nb / nn);
    *m2 = m2a + m2b + d * d * (na * nb / nn);
}

/* ------------------------------------------------------------------ */
/* Storage codec (this file's own)                                      */
/* ------------------------------------------------------------------ */

/* bfloat16 -> binary64, exact: the 16 stored bits are the upper half of a
 * binary32 pattern. */
void orc_bf16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)in[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = (double)f;
    }
}

/* binary64 -> bfloat16, round to nearest, ties to even, in ONE rounding
 * step (no intermediate binary32 rounding).  bfloat16 has 8 significant
 * bits and binary32's exponent range: the spacing of representable values
 * near |v| in [2^k, 2^(k+1)) is 2^(k-7), and 2^-133 below 2^-126
 * (subnormals).  Values whose rounded magnitude exceeds the largest finite
 * bfloat16 become infinity; NaN becomes a quiet NaN with the same sign. */
static uint16_t bf16_round_one(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);           /* a = m * 2^e, 0.5 <= m < 1 */
    int k = e - 1;                /* 2^k <= a < 2^(k+1)        */
    if (k < -126) k = -126;       /* subnormal spacing          */
    int q = k - 7;                /* spacing exponent           */
    double scaled = ldexp(a, -q); /* exact: a power-of-two scale */
    double r = nearbyint(scaled); /* default mode: ties to even  */
    double rv = ldexp(r, q);
    const double BF16_MAX = 3.38953138925153547590470800371487866880e38;
    if (rv > BF16_MAX) return (uint16_t)(sign | 0x7F80u);
    float f = (float)rv;          /* exact: rv is a bfloat16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void orc_bf16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round_one(in[i]);
}

/* IEEE binary16 -> binary64, exact: 1 sign, 5 exponent (bias 15) and 10
 * fraction bits; exponent 0 holds zero and the subnormals (fraction *
 * 2^-24), exponent 31 infinity and NaN. */
void orc_f16_decode(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        unsigned u = in[i];
        double sgn = (u & 0x8000u) ? -1.0 : 1.0;
        unsigned ex = (u >> 10) & 0x1Fu, fr = u & 0x3FFu;
        double v;
        if (ex == 0) v = ldexp((double)fr, -24);
        else if (ex == 31) v = fr ? NAN : INFINITY;
        else v = ldexp((double)(1024u + fr), (int)ex - 25);
        out[i] = sgn * v;
    }
}

/* binary64 -> binary16, round to nearest, ties to even, in one step.
 * binary16 has 11 significant bits: the spacing near |v| in [2^k, 2^(k+1))
 * is 2^(k-10), and 2^-24 below 2^-14 (subnormals).  Values whose rounded
 * magnitude exceeds the largest finite value 65504 become infinity; NaN
 * becomes a quiet NaN with the same sign. */
static uint16_t f16_round_one(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);            /* 2^(e-1) <= a < 2^e          */
    int k = e - 1;
    if (k < -14) k = -14;          /* subnormal spacing           */
    int q = k - 10;                /* spacing exponent            */
    double r = nearbyint(ldexp(a, -q));   /* exact scale, then RNE */
    double rv = ldexp(r, q);
    if (rv > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (rv < 0x1p-14)              /* subnormal (or rounded to 0)  */
        return (uint16_t)(sign | (uint16_t)ldexp(rv, 24));
    int er;
    (void)frexp(rv, &er);          /* rounding may have carried    */
    int kr = er - 1;
    unsigned frac = (unsigned)(ldexp(rv, 10 - kr) - 1024.0);
    return (uint16_t)(sign | (unsigned)(kr + 15) << 10 | frac);
}

void orc_f16_encode(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f16_round_one(in[i]);
}

/* binary64 -> binary32 with the C conversion (round to nearest even). */
void orc_f32_encode(const double *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = (float)in[i];
}

/* Threads the OpenMP loops use from now on (the CPU baseline's 1-thread
 * run); n <= 0 leaves the setting unchanged. */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
