/*
 * oracle.c -- plain CPU reference for the projection Y[M,N] = X[M,K] . W[N,K]^T
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the HIP library.
 *
 * What it follows (pages of the blog series "On descend d'un cran"):
 *   - "On descend d'un cran" (post 0), section "Ce qu'il y aura dans le
 *     depot": weights and activations are bf16, accumulators f32, nothing is
 *     quantised.
 *   - "#002 le meme compilateur sur un GPU", section "Le contrat numerique":
 *     two correct engines differ only by the order in which they add, so the
 *     reference is the exact sum, not one particular summation order.
 *   - "#004 the same compiler on Apple's chips", opening sections: add, mul
 *     and FMA are IEEE-rounded (no fast-math), and a bf16 result is rounded
 *     once, where the Hugging Face reference rounds.
 *
 * The projection has a plain definition, so this file is that definition:
 *   ref[m][n] = sum_k x[m][k] * w[n][k], exact in R.
 * Steps:
 *   1. widen every bf16 to double (exact: a bf16 is the top half of an f32);
 *   2. for each (m, n), add x*w over k in ascending order in double.  Each
 *      product of two bf16 values is exact in double (8 x 8 significand bits),
 *      and the double sum is within K * 2^-53 * sum|x*w| of the exact value;
 *   3. round the double once to f32 (the C cast, IEEE round-to-nearest-even)
 *      or once to bf16 (oracle_f64_to_bf16 below, written from the IEEE
 *      definition; no f32 intermediate, so no double rounding).
 * No blocking, no SIMD, no BLAS.  OpenMP only distributes independent
 * outputs over threads; it changes no arithmetic.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> double.  A bf16 is the high 16 bits of an IEEE f32. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * double -> bf16 bit pattern, round to nearest, ties to even (IEEE 754).
 * bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored significand bits.
 * The quantum (spacing) of bf16 numbers in the binade [2^e, 2^(e+1)) is
 * 2^(e-7) for e >= -126; below 2^-126 (subnormals) it stays 2^-133.
 * Finite results of magnitude >= 2^128 overflow to infinity.
 */
uint16_t oracle_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);          /* quiet NaN */
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;                                /* keeps -0 */

    int e2;
    frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;              /* a in [2^e, 2^(e+1)) */
    int qexp = (e < -126 ? -126 : e) - 7;
    double r = ldexp(a, -qexp);  /* a / quantum, exact (power-of-two scale) */
    double n = floor(r);
    double frac = r - n;         /* exact: r and n share the binade scale */
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0))
        n += 1.0;
    double v = ldexp(n, qexp);   /* the rounded magnitude, exact */
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    if (v < ldexp(1.0, -126)) {                     /* subnormal (or zero) */
        uint32_t mant = (uint32_t)ldexp(v, 133);    /* multiples of 2^-133 */
        return (uint16_t)(sign | mant);
    }
    int ev2;
    frexp(v, &ev2);
    int ev = ev2 - 1;                               /* v in [2^ev, 2^(ev+1)) */
    uint32_t mant = (uint32_t)(ldexp(v, 7 - ev) - 128.0);  /* 7 fraction bits */
    uint32_t bexp = (uint32_t)(ev + 127);
    return (uint16_t)(sign | (bexp << 7) | mant);
}

/* double -> f32, IEEE round-to-nearest-even (the C conversion). */
float oracle_f64_to_f32(double x)
{
    return (float)x;
}

/* One output: sum over k ascending of x[k]*w[k], in double. */
static double dot_bf16_f64(const uint16_t *x, const uint16_t *w, int64_t K)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += oracle_bf16_to_f64(x[k]) * oracle_bf16_to_f64(w[k]);
    return acc;
}

static void set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

/*
 * Y[m*N + n] = sum_k X[m*K + k] * W[n*K + k]   (all row-major, bf16 bits in,
 * double out).  threads <= 0 keeps the OpenMP default.
 */
void oracle_matmul(const uint16_t *X, const uint16_t *W, int64_t M, int64_t N,
                   int64_t K, double *Y, int threads)
{
    set_threads(threads);
    int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        Y[i] = dot_bf16_f64(X + m * K, W + n * K, K);
    }
}

/*
 * Same definition for a subset of rows: Y[j*N + n] is row rows[j] of the full
 * product.  X is the full [*, K] matrix; rows[] index into it.
 */
void oracle_matmul_rows(const uint16_t *X, const int64_t *rows, int64_t nrows,
                        const uint16_t *W, int64_t N, int64_t K, double *Y,
                        int threads)
{
    set_threads(threads);
    int64_t total = nrows * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t j = i / N, n = i % N;
        Y[i] = dot_bf16_f64(X + rows[j] * K, W + n * K, K);
    }
}

/* Element-wise final rounding of a double result. */
void oracle_round_f32(const double *in, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_f32(in[i]);
}

void oracle_round_bf16(const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16(in[i]);
}

/* f32 -> bf16 through the same IEEE rounding (an f32 is exact in double). */
void oracle_round_f32_to_bf16(const float *in, uint16_t *out, int64_t n,
                              int threads)
{
    set_threads(threads);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f64_to_bf16((double)in[i]);
}

/*
 * SwiGLU of a gate_up projection, in fp64 ("#004 the same compiler on Apple's
 * chips", section "Decode": the SwiGLU folded into the gate_up projection;
 * "#002 le meme compilateur sur un GPU", section "Emettre pour un GPU": the
 * activation fused with the projection that feeds it).  Reading of the layout
 * (the pages name the fused matrix, not its row order): rows [0, N/2) of W are
 * the gate projection and rows [N/2, N) the up projection, so with Y the fp64
 * product [M, N]:
 *     H[m][j] = silu(Y[m][j]) * Y[m][N/2 + j],   silu(g) = g / (1 + exp(-g)),
 * for j < N/2, computed in double from the (unrounded) double sums.
 */
void oracle_swiglu(const double *Y, int64_t M, int64_t N, double *H)
{
    const int64_t half = N / 2;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < half; ++j) {
            const double g = Y[m * N + j];
            const double u = Y[m * N + half + j];
            H[m * half + j] = g / (1.0 + exp(-g)) * u;
        }
}

/*
 * RMSNorm of each row of X, in double ("#004 the same compiler on Apple's
 * chips", section "Decode": the norm folded into the projection that follows
 * it).  Reading of the norm (the pages name it, not its formula): per row,
 *     r = 1 / sqrt((1/K) sum_k x_k^2 + eps),   xn_k = x_k * r * gamma_k,
 * gamma given as f32 values; computed here exactly from the inputs (the sum of
 * squares in ascending k), no rounding to bf16.
 */
void oracle_rmsnorm(const uint16_t *X, const float *gamma, int64_t M, int64_t K,
                    double eps, double *Xn)
{
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double v = oracle_bf16_to_f64(X[m * K + k]);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t k = 0; k < K; ++k)
            Xn[m * K + k] = oracle_bf16_to_f64(X[m * K + k]) * r * (double)gamma[k];
    }
}

/*
 * The projection of the RMS-normalised rows: Y[m][n] = sum_k xn[m][k] w[n][k]
 * with xn from oracle_rmsnorm, k ascending, in double.  With absolute != 0 it
 * returns sum_k |xn[m][k] w[n][k]| instead (the scale of the terms, for
 * the acceptance rule).
 */
void oracle_rmsnorm_matmul(const uint16_t *X, const float *gamma, const uint16_t *W,
                           int64_t M, int64_t N, int64_t K, double eps, int absolute,
                           double *Y, int threads)
{
    double *Xn = (double *)malloc((size_t)(M > 0 ? M : 1) * (size_t)(K > 0 ? K : 1) * sizeof(double));
    if (!Xn) return;
    oracle_rmsnorm(X, gamma, M, K, eps, Xn);
    set_threads(threads);
    int64_t total = M * N;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        const int64_t m = i / N, n = i % N;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double t = Xn[m * K + k] * oracle_bf16_to_f64(W[n * K + k]);
            acc += absolute ? fabs(t) : t;
        }
        Y[i] = acc;
    }
    free(Xn);
}

/* Number of threads an OpenMP parallel region would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
