/*
 * CPU oracle for the TN half-precision GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg
 * of bench.py may load this library.  The GPU library never links or calls it,
 * and it shares no code, header or table with the GPU library.
 *
 * What it computes (the plain definition, nothing more):
 *
 *     C[i*ldc + j] = fp16_rne( sum_{k=0}^{K-1} A[i*lda + k] * B[j*ldb + k] )
 *
 * for 0 <= i < M, 0 <= j < N, with A an M x K row-major matrix and B a K x N
 * column-major matrix (stored as N rows of K halves), both binary16.
 * Sources for the operation:
 *   - "RL驱动CUDA L2 GEMM内核自动调优：A100/H100 tile size与融合优化"
 *     (blog.hotdry.top, 2025-12-05), 正文 paragraph 1: the kernel is a
 *     half-precision GEMM (HGEMM); paragraph 3: A is row-major and B is
 *     column-major, and the kernel family name ends in "TN".
 *   - same page, 集成步骤 / correctness paragraph: results are judged by
 *     relative error against a library GEMM, so the oracle is the exact
 *     definition, rounded once.
 * Readings where the pages are silent:
 *   - the sum is taken in binary64 in index order k = 0..K-1, one result per
 *     (i, j); every product of two binary16 values is exact in binary64
 *     (11-bit x 11-bit significands), so the only roundings are the K-1
 *     binary64 additions and the final binary16 rounding;
 *   - alpha = 1, beta = 0: C is written, never read; K = 0 gives +0;
 *   - C is row-major with leading dimension ldc >= N;
 *   - binary16 rounding is IEEE round-to-nearest, ties-to-even; magnitudes at
 *     or above 65520 become infinity; NaN stays NaN.
 *
 * The binary16 decoder and encoder below are written from the IEEE 754
 * binary16 format (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits;
 * exponent field 0 encodes zero and subnormals m * 2^-24, field 31 encodes
 * infinity and NaN).  No half-precision hardware arithmetic is used.
 *
 * The int8 variant (ref_igemm_tn): the INT8 mode of the same page's
 * multi-precision scheduling (正文 paragraph 3, FP16/INT8 switching).  The page
 * leaves its result type open; the reading taken is the exact integer sum
 *
 *     C[i*ldc + j] = sum_{k=0}^{K-1} A[i*lda + k] * B[j*ldb + k]
 *
 * over int8 operands, stored as int32 (a sum that does not fit int32 is
 * reported, not wrapped).
 *
 * The overlap micro-benchmark's arithmetic (ref_fma_chain): "B-08. Hopper TMA：
 * 从单线程 Bulk Copy 到吞吐墙" (lqnn.cn) §5 sweeps a number of FMA iterations per
 * loaded element; here each element becomes y = x, then fma_iters times
 * y = fmaf(y, alpha, beta), with C99 fmaf (one rounding to binary32 per step).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see oracle/__init__.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- codec -- */

/* binary16 bit pattern -> the exact binary64 value it encodes. */
double ref_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);                 /* zero, subnormal */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;                    /* NaN, infinity */
    } else {
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative binary64 value q (< 2^52) to an integer, ties to even. */
static double round_half_even(double q)
{
    const double fl = floor(q);
    const double rem = q - fl; /* exact: q and fl share the binade or fl == 0 */
    if (rem > 0.5) return fl + 1.0;
    if (rem < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary64 value -> nearest binary16 bit pattern, ties to even. */
uint16_t ref_f64_to_f16(double x)
{
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    const double a = fabs(x);
    /* 65504 is the largest finite value; the midpoint to 2^16 is 65520 and
       65504 has an odd fraction, so the tie goes up to infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;               /* 2^e <= a < 2^(e+1) */
    if (e < -14) {
        /* subnormal range: the quantum is 2^-24 */
        const double n = round_half_even(ldexp(a, 24));
        /* n == 1024 lands exactly on the smallest normal, whose bit pattern
           is 0x0400 == 1024: the subnormal formula covers it. */
        return (uint16_t)(sign | (uint16_t)n);
    }
    double n = round_half_even(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

void ref_f16_to_f64_array(const uint16_t* in, double* out, int64_t n)
{
    for (int64_t t = 0; t < n; ++t) out[t] = ref_f16_to_f64(in[t]);
}

void ref_f64_to_f16_array(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t t = 0; t < n; ++t) out[t] = ref_f64_to_f16(in[t]);
}

/* ----------------------------------------------------------------- GEMM -- */

/* Decoding table for all 65536 binary16 patterns, filled from ref_f16_to_f64. */
static double g_dec[65536];
static int g_dec_ready = 0;

static void ensure_table(void)
{
    if (g_dec_ready) return;
    for (int h = 0; h < 65536; ++h) g_dec[h] = ref_f16_to_f64((uint16_t)h);
    g_dec_ready = 1;
}

/* sum_{k=0}^{K-1} a[k] * b[k] in binary64, in index order. */
static double dot_in_order(const uint16_t* a, const uint16_t* b, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += g_dec[a[k]] * g_dec[b[k]];
    return s;
}

/* Full product: every element of C.  Returns 0, or -1 on a bad argument. */
int ref_hgemm_tn(int64_t M, int64_t N, int64_t K,
                 const uint16_t* A, int64_t lda,
                 const uint16_t* B, int64_t ldb,
                 uint16_t* C, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N) return -1;
    ensure_table();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            C[i * ldc + j] = ref_f64_to_f16(dot_in_order(A + i * lda, B + j * ldb, K));
    return 0;
}

/* Selected elements only: out[t] = C[rows[t], cols[t]] (binary16 bits) and,
   when sums != NULL, sums[t] = the unrounded binary64 sum. */
int ref_hgemm_tn_entries(int64_t M, int64_t N, int64_t K,
                         const uint16_t* A, int64_t lda,
                         const uint16_t* B, int64_t ldb,
                         int64_t count, const int64_t* rows, const int64_t* cols,
                         uint16_t* out, double* sums)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    ensure_table();
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const double s = dot_in_order(A + rows[t] * lda, B + cols[t] * ldb, K);
        out[t] = ref_f64_to_f16(s);
        if (sums) sums[t] = s;
    }
    return 0;
}

/* ------------------------------------------------------------ int8 GEMM -- */

/* sum_{k=0}^{K-1} a[k] * b[k], exact in int64 (|sum| <= K * 2^14). */
static int64_t idot(const int8_t* a, const int8_t* b, int64_t K)
{
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += (int64_t)a[k] * (int64_t)b[k];
    return s;
}

static int fits_int32(int64_t s) { return s >= INT32_MIN && s <= INT32_MAX; }

/* Full int8 product.  Returns 0; -1 on a bad argument; -2 when some sum does
   not fit int32 (C is then incomplete). */
int ref_igemm_tn(int64_t M, int64_t N, int64_t K,
                 const int8_t* A, int64_t lda,
                 const int8_t* B, int64_t ldb,
                 int32_t* C, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || ldc < N) return -1;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(|:bad)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            const int64_t s = idot(A + i * lda, B + j * ldb, K);
            if (fits_int32(s)) C[i * ldc + j] = (int32_t)s;
            else bad = 1;
        }
    return bad ? -2 : 0;
}

/* Selected elements of the int8 product: out[t] = C[rows[t], cols[t]]. */
int ref_igemm_tn_entries(int64_t M, int64_t N, int64_t K,
                         const int8_t* A, int64_t lda,
                         const int8_t* B, int64_t ldb,
                         int64_t count, const int64_t* rows, const int64_t* cols,
                         int32_t* out)
{
    if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || count < 0) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t s = idot(A + rows[t] * lda, B + cols[t] * ldb, K);
        if (fits_int32(s)) out[t] = (int32_t)s;
        else bad = 1;
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------ overlap arithmetic -- */

/* out[i] = x[i] after fma_iters steps of y = fmaf(y, alpha, beta). */
int ref_fma_chain(const float* x, float* out, int64_t n, int32_t fma_iters, float alpha,
                  float beta)
{
    if (n < 0 || fma_iters < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float y = x[i];
        for (int32_t it = 0; it < fma_iters; ++it) y = fmaf(y, alpha, beta);
        out[i] = y;
    }
    return 0;
}

/* Threads an OpenMP parallel region of this library uses. */
int ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the threads of this library's later parallel regions (n >= 1): the
   environment does not always reach the OpenMP runtime this library links. */
void ref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
