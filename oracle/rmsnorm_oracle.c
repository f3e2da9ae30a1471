/*
 * rmsnorm_oracle.c -- plain, slow, fp64 CPU oracle for the row RMSNorm forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP library; the dtype codes below are restated here on purpose.
 *
 * What it computes, per row m of an [M, N] row-major matrix x and a weight w[N]:
 *
 *     ss        = sum_j x[m,j]^2                       (fp64, sequential j)
 *     ms        = ss / N                                (the true column count)
 *     rstd[m]   = 1 / sqrt(ms + eps)                    (fp64, not rounded)
 *     y[m,j]    = round_dtype( x[m,j] * rstd[m] * (offset + w[j]) )
 *
 * Sources:
 *   - "Rmsnorm Kernel Optimization", section "Overview": the normalisation is x
 *     divided by the root of (mean of x squared plus eps), times the weight.
 *   - "Why cutile's rmsnorm required full register", kernel listing in the
 *     opening report: the weight enters as (offset + w) with offset 0.0 for
 *     Llama and 1.0 for Gemma3; the mean divides by the real width N, not by
 *     the padded tile width; eps and offset are fp32 constants; the per-row
 *     reciprocal root is written out as rstd; y is cast to the input dtype once,
 *     at the end.
 *   - "Rmsnorm Kernel Optimization", section "Key Optimizations" / "Common
 *     Pitfalls": the reduction must not run in the 16-bit input type.  Here it
 *     runs in fp64, well beyond the fp32 the GPU path uses.
 *
 * The backward below is derived by differentiating this forward (the pages
 * keep rstd for a backward pass but do not print one).
 *
 * Readings taken where the pages are silent:
 *   - eps and offset arrive as fp32 (as in the listing) and are widened exactly.
 *   - The final cast is IEEE round-to-nearest-even, applied once, directly from
 *     fp64 to the 16-bit format, with gradual underflow (subnormals kept) and
 *     overflow to infinity.
 *   - w has the same 16-bit dtype as x.
 *
 * The 16-bit codecs below are written from the IEEE-754 binary16 format
 * (1 sign, 5 exponent, 10 fraction bits, bias 15) and the bfloat16 format
 * (1 sign, 8 exponent, 7 fraction bits, bias 127: the top half of binary32).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of this oracle's own interface */
#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* Field widths of a 16-bit IEEE-style format. */
typedef struct {
    int exp_bits;   /* E */
    int frac_bits;  /* P */
} fmt16;

static fmt16 fmt_of(int dtype)
{
    fmt16 f;
    if (dtype == ORACLE_BF16) { f.exp_bits = 8; f.frac_bits = 7; }
    else                      { f.exp_bits = 5; f.frac_bits = 10; }
    return f;
}

/* Exact value of a 16-bit pattern. */
double oracle_decode(uint16_t bits, int dtype)
{
    const fmt16 f = fmt_of(dtype);
    const int bias = (1 << (f.exp_bits - 1)) - 1;
    const unsigned sign = bits >> 15;
    const unsigned e = (bits >> f.frac_bits) & ((1u << f.exp_bits) - 1u);
    const unsigned frac = bits & ((1u << f.frac_bits) - 1u);
    double mag;
    if (e == (1u << f.exp_bits) - 1u) {
        mag = frac ? NAN : INFINITY;
    } else if (e == 0) {
        /* subnormal: frac * 2^(1 - bias - P) */
        mag = ldexp((double)frac, 1 - bias - f.frac_bits);
    } else {
        /* normal: (2^P + frac) * 2^(e - bias - P) */
        mag = ldexp((double)((1u << f.frac_bits) + frac), (int)e - bias - f.frac_bits);
    }
    return sign ? -mag : mag;
}

/*
 * Round a double to the nearest 16-bit value, ties to even, in one step.
 *
 * For |v| with unbiased exponent ex (clamped below at emin = 1 - bias so that
 * the subnormal range shares emin's quantum), the representable values near |v|
 * are the integer multiples n of q = 2^(ex - P).  s = |v| / q is exact in fp64
 * (a power-of-two scaling) and lies below 2^(P+1); n = s rounded to the nearest
 * integer, ties to the even n.  Because the bit patterns of a binary format
 * are ordered like the magnitudes, the pattern is ((ex - emin) << P) + n; a
 * carry out of the fraction lands on the next binade, and a pattern at or past
 * the all-ones exponent is infinity.
 */
uint16_t oracle_encode_rne(double v, int dtype)
{
    const fmt16 f = fmt_of(dtype);
    const int bias = (1 << (f.exp_bits - 1)) - 1;
    const int emin = 1 - bias;
    const uint32_t inf_bits = ((1u << f.exp_bits) - 1u) << f.frac_bits;
    const uint32_t sign = signbit(v) ? 0x8000u : 0u;

    if (isnan(v))
        return (uint16_t)(sign | inf_bits | (1u << (f.frac_bits - 1))); /* quiet NaN */
    double a = fabs(v);
    if (a == 0.0)
        return (uint16_t)sign;
    if (isinf(a))
        return (uint16_t)(sign | inf_bits);

    int k;
    (void)frexp(a, &k);            /* a = m * 2^k, m in [0.5, 1) */
    int ex = k - 1;                /* a in [2^ex, 2^(ex+1)) */
    if (ex < emin) ex = emin;
    /* far above the largest binade: certainly infinity (also keeps ldexp exact) */
    if (ex > bias + 1)
        return (uint16_t)(sign | inf_bits);

    const double s = ldexp(a, f.frac_bits - ex);   /* exact, s < 2^(P+1) */
    double n = floor(s);
    const double r = s - n;                        /* exact */
    if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;

    uint32_t bits = ((uint32_t)(ex - emin) << f.frac_bits) + (uint32_t)n;
    if (bits >= inf_bits)
        bits = inf_bits;
    return (uint16_t)(sign | bits);
}

void oracle_decode_array(const uint16_t* bits, double* out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode(bits[i], dtype);
}

void oracle_encode_array(const double* v, uint16_t* out, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_rne(v[i], dtype);
}

/*
 * Row RMSNorm forward, fp64.  Returns 0, or -1 on an argument it cannot take.
 *   x       [M*N] 16-bit patterns, row-major
 *   w       [N]   16-bit patterns, same dtype as x
 *   eps     fp32 epsilon, added to the mean of squares inside the root
 *   offset  fp32 offset added to every weight (0.0 Llama, 1.0 Gemma3)
 *   y       [M*N] output patterns, rounded once to the dtype
 *   rstd    [M]   fp64 1/sqrt(mean + eps), unrounded
 *   y_exact [M*N] fp64 value before the final rounding (may be NULL)
 */
int oracle_rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                       float eps, float offset, int dtype,
                       uint16_t* y, double* rstd, double* y_exact)
{
    if (M < 0 || N <= 0) return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return -1;
    const double e = (double)eps;
    const double off = (double)offset;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double xv = oracle_decode(xr[j], dtype);
            ss += xv * xv;
        }
        const double ms = ss / (double)N;
        const double r = 1.0 / sqrt(ms + e);
        rstd[m] = r;
        for (int64_t j = 0; j < N; ++j) {
            const double xv = oracle_decode(xr[j], dtype);
            const double ye = xv * r * (off + oracle_decode(w[j], dtype));
            y[m * N + j] = oracle_encode_rne(ye, dtype);
            if (y_exact) y_exact[m * N + j] = ye;
        }
    }
    return 0;
}

/*
 * Forward in fp64 on fp64 inputs, with no 16-bit codec on either side: the
 * same formula as oracle_rmsnorm_fwd.  It exists so that the backward can be
 * checked by finite differences of the forward on perturbed inputs.
 *   x [M*N], w [N] fp64; y [M*N] and rstd [M] fp64 outputs.
 */
int oracle_rmsnorm_fwd_f64(const double* x, const double* w, int64_t M, int64_t N,
                           double eps, double offset, double* y, double* rstd)
{
    if (M < 0 || N <= 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const double* xr = x + m * N;
        double ss = 0.0;
        for (int64_t j = 0; j < N; ++j) ss += xr[j] * xr[j];
        const double r = 1.0 / sqrt(ss / (double)N + eps);
        rstd[m] = r;
        for (int64_t j = 0; j < N; ++j) y[m * N + j] = xr[j] * r * (offset + w[j]);
    }
    return 0;
}

/*
 * Row RMSNorm backward, fp64.  The pages store rstd for a backward pass
 * ("Why cutile's rmsnorm required full register", kernel listing) but give
 * no formula; this one follows from differentiating the forward.  With
 * g_j = offset + w_j, r = rstd[m] and y_j = x_j r g_j, where
 * r = (mean_j x_j^2 + eps)^(-1/2) so that dr/dx_k = -r^3 x_k / N:
 *
 *     c[m]     = (1/N) sum_j dy[m,j] g_j x[m,j]
 *     dx[m,k]  = r (g_k dy[m,k] - r^2 c[m] x[m,k])
 *     dw[j]    = sum_m dy[m,j] x[m,j] r[m]          (d g_j / d w_j = 1)
 *
 *   x, dy   [M*N] 16-bit patterns; w [N] patterns (same dtype)
 *   rstd    [M] fp64 (the forward's rstd, given, not recomputed)
 *   offset  fp32, as in the forward
 *   dx      [M*N] patterns, rounded once to the dtype (nearest even)
 *   dw      [N] fp64, unrounded
 *   dx_exact [M*N] fp64 before rounding (may be NULL)
 *   dx_scale [M*N] fp64 (may be NULL): |r g_k dy_k| + |r^3 x_k| (1/N) sum_j |dy_j g_j x_j|,
 *            the size of the terms dx is computed from, for error bounds
 *   dw_scale [N]   fp64 (may be NULL): sum_m |dy x r|, likewise
 */
int oracle_rmsnorm_bwd(const uint16_t* x, const uint16_t* w, const uint16_t* dy,
                       const double* rstd, int64_t M, int64_t N, float offset, int dtype,
                       uint16_t* dx, double* dw, double* dx_exact, double* dx_scale,
                       double* dw_scale)
{
    if (M < 0 || N <= 0) return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return -1;
    const double off = (double)offset;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * N;
        const uint16_t* dyr = dy + m * N;
        const double r = rstd[m];
        double c = 0.0, cabs = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double t = oracle_decode(dyr[j], dtype) * (off + oracle_decode(w[j], dtype)) *
                             oracle_decode(xr[j], dtype);
            c += t;
            cabs += fabs(t);
        }
        c /= (double)N;
        cabs /= (double)N;
        for (int64_t k = 0; k < N; ++k) {
            const double xk = oracle_decode(xr[k], dtype);
            const double gk = off + oracle_decode(w[k], dtype);
            const double dyk = oracle_decode(dyr[k], dtype);
            const double v = r * (gk * dyk - r * r * c * xk);
            dx[m * N + k] = oracle_encode_rne(v, dtype);
            if (dx_exact) dx_exact[m * N + k] = v;
            if (dx_scale) dx_scale[m * N + k] = fabs(r * gk * dyk) + fabs(r * r * r * xk) * cabs;
        }
    }

    /* dw: each column summed over rows in increasing m; columns are taken in
     * chunks so that the rows are walked in memory order */
    const int64_t CH = 64;
#pragma omp parallel for schedule(static)
    for (int64_t j0 = 0; j0 < N; j0 += CH) {
        const int64_t j1 = j0 + CH < N ? j0 + CH : N;
        double acc[64], aabs[64];
        for (int64_t j = j0; j < j1; ++j) { acc[j - j0] = 0.0; aabs[j - j0] = 0.0; }
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t j = j0; j < j1; ++j) {
                const double t = oracle_decode(dy[m * N + j], dtype) * oracle_decode(x[m * N + j], dtype) *
                                 rstd[m];
                acc[j - j0] += t;
                aabs[j - j0] += fabs(t);
            }
        }
        for (int64_t j = j0; j < j1; ++j) {
            dw[j] = acc[j - j0];
            if (dw_scale) dw_scale[j] = aabs[j - j0];
        }
    }
    return 0;
}

/*
 * The same backward on fp64 inputs with no codec on either side, for inputs
 * of a wider type (fp32 values widen to fp64 exactly).  Same formula and
 * summation order as oracle_rmsnorm_bwd; dx is returned unrounded.
 *   x, dy [M*N] fp64; w [N] fp64; rstd [M] fp64; offset fp64 (an fp32 value)
 *   dx_exact [M*N], dw [N] fp64 outputs; dx_scale [M*N], dw_scale [N] as above
 *   (either may be NULL)
 */
int oracle_rmsnorm_bwd_f64(const double* x, const double* w, const double* dy, const double* rstd,
                           int64_t M, int64_t N, double offset, double* dx_exact, double* dw,
                           double* dx_scale, double* dw_scale)
{
    if (M < 0 || N <= 0) return -1;

#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const double* xr = x + m * N;
        const double* dyr = dy + m * N;
        const double r = rstd[m];
        double c = 0.0, cabs = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double t = dyr[j] * (offset + w[j]) * xr[j];
            c += t;
            cabs += fabs(t);
        }
        c /= (double)N;
        cabs /= (double)N;
        for (int64_t k = 0; k < N; ++k) {
            const double gk = offset + w[k];
            const double v = r * (gk * dyr[k] - r * r * c * xr[k]);
            dx_exact[m * N + k] = v;
            if (dx_scale) dx_scale[m * N + k] = fabs(r * gk * dyr[k]) + fabs(r * r * r * xr[k]) * cabs;
        }
    }

    for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0, aabs = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            const double t = dy[m * N + j] * x[m * N + j] * rstd[m];
            acc += t;
            aabs += fabs(t);
        }
        dw[j] = acc;
        if (dw_scale) dw_scale[j] = aabs;
    }
    return 0;
}

/* Threads the OpenMP loops use from now on (n >= 1); a timing knob only, the
   results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads the OpenMP loop above will use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
