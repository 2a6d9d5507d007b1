/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the dense
 * half-precision GEMM C = A * B.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares a line of code with it.
 *
 * What it follows:
 *   - "Xe2 ESIMD GEMM" page, section "Correctness testing": the GPU result of
 *     an FP16 GEMM is judged against an FP32 CPU reference.  Here the
 *     reference accumulates in fp64 and rounds once to fp32 at the end, so
 *     the only error left in it is that one rounding.
 *   - The operation itself is the textbook matrix product
 *         C[b][i][j] = sum_{k=0}^{K-1} A[b][i][k] * B[b][k][j]
 *     with row-major A (M x K, leading dimension lda), row-major B (K x N,
 *     leading dimension ldb; the page calls this layout B_T[K,N], section
 *     "Sample code") and row-major C (M x N, leading dimension ldc).
 *
 * Inputs are IEEE binary16 (fp16) or bfloat16 (bf16) BIT PATTERNS, i.e. the
 * exact values the GPU reads.  They are decoded exactly to double by this
 * file's own bit-level decoders.  Every product of two 16-bit values is exact
 * in double (at most 11+11 significant bits), so the only rounding inside the
 * sum is fp64 addition, performed in ascending k.
 *
 * The same file holds the reference for the second workload, scaled
 * dot-product attention (oracle_attention, below).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: the summation order
 * written below must be the one executed).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Exact decoders                                                      */
/* ------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent field 0 is zero/subnormal (value f * 2^-24), 31 is
 * infinity (f == 0) or NaN. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);          /* f * 2^(-126-7) */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134); /* 1.f * 2^(e-127) */
    return sign ? -v : v;
}

void oracle_decode_f16(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f16_to_f64(src[i]);
}

void oracle_decode_bf16(const uint16_t *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_bf16_to_f64(src[i]);
}

/* ------------------------------------------------------------------ */
/* Round-to-nearest-even encoders (for the 16-bit output forms)        */
/* ------------------------------------------------------------------ */

/* Round a finite non-negative double x to the nearest integer, ties to
 * even, without relying on the floating-point environment. */
static double round_half_even(double x)
{
    double fl = floor(x);
    double diff = x - fl;               /* exact: x and fl are close */
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp32 value -> binary16 bits, round to nearest, ties to even.
 * The quantum of binary16 in binade [2^e, 2^(e+1)) is 2^(e-10) for
 * e >= -14 and 2^-24 for all subnormals.  Values that round to 2^16 or
 * more become infinity. */
uint16_t oracle_f32_to_f16(float xf)
{
    double x = (double)xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7e00;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7c00;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                       /* a = m * 2^e, m in [0.5, 1) */
    e -= 1;                             /* a in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;               /* subnormal range shares quantum 2^-24 */
    double q = ldexp(1.0, e - 10);
    double n = round_half_even(a / q);  /* a/q exact: power-of-two scale */
    double r = n * q;
    if (r >= 65536.0) return sign | 0x7c00;
    /* encode r exactly */
    if (r < ldexp(1.0, -14)) {          /* subnormal (or rounded to zero) */
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    }
    int re;
    frexp(r, &re);
    re -= 1;                            /* r in [2^re, 2^(re+1)) */
    uint16_t frac = (uint16_t)(r / ldexp(1.0, re - 10) - 1024.0);
    return sign | (uint16_t)((re + 15) << 10) | frac;
}

/* fp32 value -> bfloat16 bits, round to nearest, ties to even.  bf16 keeps
 * 8 significant bits with the fp32 exponent range; the quantum in binade
 * [2^e, 2^(e+1)) is 2^(e-7) for e >= -126 and 2^-133 below. */
uint16_t oracle_f32_to_bf16(float xf)
{
    double x = (double)xf;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7fc0;
    double a = fabs(x);
    if (isinf(a)) return sign | 0x7f80;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    e -= 1;
    if (e < -126) e = -126;
    double q = ldexp(1.0, e - 7);
    double n = round_half_even(a / q);
    double r = n * q;
    if (r >= ldexp(1.0, 128)) return sign | 0x7f80;
    if (r < ldexp(1.0, -126)) {
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    }
    int re;
    frexp(r, &re);
    re -= 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, re - 7) - 128.0);
    return sign | (uint16_t)((re + 127) << 7) | frac;
}

void oracle_encode_f16(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f32_to_f16(src[i]);
}

void oracle_encode_bf16(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f32_to_bf16(src[i]);
}

/* ------------------------------------------------------------------ */
/* The product                                                         */
/* ------------------------------------------------------------------ */

static double decode(int is_bf16, uint16_t h)
{
    return is_bf16 ? oracle_bf16_to_f64(h) : oracle_f16_to_f64(h);
}

/*
 * oracle_gemm: for every batch b, row i and column j
 *     acc = 0 (fp64);  for k = 0 .. K-1 ascending: acc += A[b][i][k]*B[b][k][j]
 *     C32[b][i][j] = (float)acc      (one rounding, to nearest even)
 *     C64[b][i][j] = acc             (when C64 != NULL)
 *
 * Loop order: rows i outside, then k ascending, then columns j.  Every
 * element's sum is still taken in ascending k, so each result equals the
 * textbook i-j-k dot product bit for bit; this order only lets the
 * inner loop stream a row of B.
 *
 * dtype: 0 = fp16 inputs, 1 = bf16 inputs.  All strides and leading
 * dimensions are in elements.  Rows (b, i) are independent and are spread
 * over OpenMP threads; nothing is shared between them.
 */
void oracle_gemm(int dtype, int64_t batch, int64_t M, int64_t N, int64_t K,
                 const uint16_t *A, int64_t lda, int64_t strideA,
                 const uint16_t *B, int64_t ldb, int64_t strideB,
                 float *C32, double *C64, int64_t ldc, int64_t strideC)
{
    int is_bf16 = (dtype == 1);
    int64_t rows = batch * M;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / M, i = r % M;
        const uint16_t *arow = A + b * strideA + i * lda;
        const uint16_t *Bb = B + b * strideB;
        double acc[256];                 /* one block of 256 columns */
        for (int64_t j0 = 0; j0 < N; j0 += 256) {
            int64_t jn = (N - j0 < 256) ? (N - j0) : 256;
            for (int64_t j = 0; j < jn; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = decode(is_bf16, arow[k]);
                const uint16_t *brow = Bb + k * ldb + j0;
                for (int64_t j = 0; j < jn; ++j)
                    acc[j] += a * decode(is_bf16, brow[j]);
            }
            for (int64_t j = 0; j < jn; ++j) {
                int64_t off = b * strideC + i * ldc + j0 + j;
                if (C32) C32[off] = (float)acc[j];
                if (C64) C64[off] = acc[j];
            }
        }
    }
}

/*
 * oracle_gemm_at: the same definition evaluated at n chosen output
 * positions (bidx[t], row[t], col[t]) as a plain dot product in ascending
 * k.  Used where the full product is too large to form on the CPU.
 */
void oracle_gemm_at(int dtype, int64_t K,
                    const uint16_t *A, int64_t lda, int64_t strideA,
                    const uint16_t *B, int64_t ldb, int64_t strideB,
                    int64_t n, const int64_t *bidx, const int64_t *row,
                    const int64_t *col, float *out32, double *out64)
{
    int is_bf16 = (dtype == 1);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *Ab = A + bidx[t] * strideA + row[t] * lda;
        const uint16_t *Bb = B + bidx[t] * strideB + col[t];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += decode(is_bf16, Ab[k]) * decode(is_bf16, Bb[k * ldb]);
        if (out32) out32[t] = (float)acc;
        if (out64) out64[t] = acc;
    }
}

/* ------------------------------------------------------------------ */
/* Scaled dot-product attention (the pages' "SDP" / flash-attention     */
/* workload): O = softmax(scale * Q K^T) V, row by row                  */
/* ------------------------------------------------------------------ */

/*
 * oracle_attention: for n chosen output rows (bh[t], row[t]) of
 *     O[b][i][d] = sum_j p_j V[b][j][d] / sum_j p_j,
 *     p_j = exp(s_j - max_j s_j),
 *     s_j = scale * sum_{e=0}^{D-1} Q[b][i][e] * K[b][j][e]
 * with j over the Skv keys, no mask.  This is the plain definition of a
 * softmax over the scaled logits followed by the weighted sum of value rows
 * (the "Xe2 Nbarrier Pipelining" page, section "Proven Pattern: SDP Kernel Split
 * Barrier B", names this kernel, an HD = 256 flash attention); subtracting
 * the row maximum changes no exact value and keeps exp() finite.
 *
 * Everything is fp64: the dot products in ascending e (the products of two
 * 16-bit values are exact), exp() from the C library, the sums over keys
 * in ascending j, one division per output.  out32 gets the result rounded
 * once to fp32, out64 (when not NULL) the fp64 value.  Output t is written
 * at out[t * D + d].  Skv == 0 writes zeros (an empty softmax has no
 * weights).  Q, K, V are 16-bit patterns, leading dimensions and batch
 * strides in elements; scale is used as given (the GPU path receives the
 * same value).
 */
void oracle_attention(int dtype, int64_t Skv, int64_t D,
                      const uint16_t *Q, int64_t ldq, int64_t strideQ,
                      const uint16_t *K, int64_t ldk, int64_t strideK,
                      const uint16_t *V, int64_t ldv, int64_t strideV,
                      double scale, int64_t n, const int64_t *bh, const int64_t *row,
                      float *out32, double *out64)
{
    int is_bf16 = (dtype == 1);
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)(Skv > 0 ? Skv : 1) * sizeof(double));
        double *q = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
        double *o = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) {
            const uint16_t *qrow = Q + bh[t] * strideQ + row[t] * ldq;
            const uint16_t *Kb = K + bh[t] * strideK;
            const uint16_t *Vb = V + bh[t] * strideV;
            for (int64_t e = 0; e < D; ++e) q[e] = decode(is_bf16, qrow[e]);
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            if (Skv > 0) {
                /* logits and their maximum */
                double smax = -INFINITY;
                for (int64_t j = 0; j < Skv; ++j) {
                    const uint16_t *krow = Kb + j * ldk;
                    double acc = 0.0;
                    for (int64_t e = 0; e < D; ++e) acc += q[e] * decode(is_bf16, krow[e]);
                    s[j] = scale * acc;
                    if (s[j] > smax) smax = s[j];
                }
                /* weights, their sum, and the weighted sum of value rows */
                double l = 0.0;
                for (int64_t j = 0; j < Skv; ++j) {
                    double pj = exp(s[j] - smax);
                    l += pj;
                    const uint16_t *vrow = Vb + j * ldv;
                    for (int64_t d = 0; d < D; ++d) o[d] += pj * decode(is_bf16, vrow[d]);
                }
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
            }
            for (int64_t d = 0; d < D; ++d) {
                if (out32) out32[t * D + d] = (float)o[d];
                if (out64) out64[t * D + d] = o[d];
            }
        }
        free(s);
        free(q);
        free(o);
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}

/* Set that number (n >= 1); the results do not depend on it, since every
 * output element is summed by one thread in its fixed order. */
void oracle_set_num_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}
