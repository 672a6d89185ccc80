/*
 * oracle.c -- plain double-precision CPU oracle for the single-precision
 * matrix product C = A x B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the HIP library.
 *
 * What it computes.  The plain definition of the product: for an M x K
 * matrix A and a K x N matrix B, entry (i, j) of C is the sum over
 * k = 0 .. K-1 of A(i,k) * B(k,j)  [article "硬件加速原理：CUDA核函数优化矩阵
 * 乘法的内存访问模式", section "矩阵乘法的计算特性" (computational properties of
 * matrix multiplication), the summation formula; also the textbook chapter
 * "4. 矩阵乘法性能优化", opening paragraph].  Storage is row-major with
 * explicit leading dimensions, as in the blog "【infra之路】03_动手写 CUDA
 * Kernel", v1 Naive kernel (A indexed row*width+k, B indexed k*width+col).
 *
 * Precision.  Inputs are IEEE single precision.  Each product of two floats
 * is formed in double, where it is exact (24 + 24 significand bits fit in
 * 53), and the products are summed in double in ascending k.  The blog's own
 * CPU check sums in float; that is deliberately not followed.  Alongside the
 * value the oracle returns S(i,j) = sum_k |A(i,k) * B(k,j)|, the scale that
 * the per-element tolerance |C - Cref| <= 1e-5 * S + 1e-6 is stated in.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -fno-fast-math -fopenmp.
 * -ffp-contract=off keeps every multiply and add separately rounded; OpenMP
 * only splits whole rows between threads, so the arithmetic of each entry is
 * the same for any thread count.
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1

static int dims_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    if (lda < (K > 1 ? K : 1)) return 0;
    if (ldb < (N > 1 ? N : 1)) return 0;
    return 1;
}

/*
 * Full product.  Cref (M x N, leading dimension ldr) receives the double sums;
 * Sabs (same shape, leading dimension lds) receives the absolute-product sums
 * and may be NULL.  Loop order i, k, j: for a fixed (i, j) the terms are
 * still added in ascending k, so each entry equals the textbook i, j, k dot
 * product bit for bit (oracle_entries_f64 below computes exactly that).
 * nthreads <= 0 lets OpenMP choose.
 */
int oracle_sgemm_f64(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     double *Cref, int64_t ldr,
                     double *Sabs, int64_t lds,
                     int nthreads)
{
    if (!dims_ok(M, N, K, lda, ldb)) return ORACLE_BAD_ARG;
    if (ldr < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (Sabs && lds < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (!Cref || (K > 0 && (!A || !B))) return ORACLE_BAD_ARG;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        double *c = Cref + i * ldr;
        double *s = Sabs ? Sabs + i * lds : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (s)
            for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *b = B + k * ldb;
            if (s) {
                for (int64_t j = 0; j < N; ++j) {
                    const double p = a * (double)b[j];
                    c[j] += p;
                    s[j] += fabs(p);
                }
            } else {
                for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[j];
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Selected entries.  For e < n, entry (I[e], J[e]) is the ascending-k dot
 * product of row I[e] of A with column J[e] of B, in double; sabs may be NULL.
 * Used where the full product would take too long on the host.
 */
int oracle_entries_f64(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       int64_t n, const int64_t *I, const int64_t *J,
                       double *cref, double *sabs)
{
    if (!dims_ok(M, N, K, lda, ldb) || n < 0) return ORACLE_BAD_ARG;
    if (n > 0 && (!I || !J || !cref)) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e)
        if (I[e] < 0 || I[e] >= M || J[e] < 0 || J[e] >= N) return ORACLE_BAD_ARG;
    if (K > 0 && n > 0 && (!A || !B)) return ORACLE_BAD_ARG;

    for (int64_t e = 0; e < n; ++e) {
        const int64_t i = I[e], j = J[e];
        double acc = 0.0, sab = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
            acc += p;
            sab += fabs(p);
        }
        cref[e] = acc;
        if (sabs) sabs[e] = sab;
    }
    return ORACLE_OK;
}

/*
 * The general form C = alpha * op(A) op(B) + beta * C0.  op(A)(i,k) is
 * A[i*lda + k], or A[k*lda + i] when transA; op(B)(k,j) is B[k*ldb + j], or
 * B[j*ldb + k] when transB.  The sum over k is formed exactly as in
 * oracle_sgemm_f64 (exact double products, ascending k, double sums); then
 * Cref = alpha * sum + beta * C0, in double.  When beta == 0, C0 is not read
 * (it may be NULL or hold NaN).  Sabs (may be NULL) receives
 * |alpha| * sum_k |op(A)(i,k) op(B)(k,j)| + |beta| * |C0(i,j)|, the scale of
 * the tolerance for this form.  The definition is the plain product's (see
 * the top of this file) with the transposed indexing spelled out above.
 */
int oracle_sgemm_ex_f64(int transA, int transB, int64_t M, int64_t N, int64_t K, double alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, double beta,
                        const float *C0, int64_t ldc0, double *Cref, int64_t ldr,
                        double *Sabs, int64_t lds, int nthreads)
{
    const int64_t acols = transA ? M : K, bcols = transB ? K : N;
    if (M < 0 || N < 0 || K < 0) return ORACLE_BAD_ARG;
    if (lda < (acols > 1 ? acols : 1) || ldb < (bcols > 1 ? bcols : 1)) return ORACLE_BAD_ARG;
    if (ldr < (N > 1 ? N : 1) || (Sabs && lds < (N > 1 ? N : 1))) return ORACLE_BAD_ARG;
    if (beta != 0.0 && ldc0 < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (!Cref || (K > 0 && (!A || !B)) || (beta != 0.0 && !C0)) return ORACLE_BAD_ARG;

#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < M; ++i) {
        double *c = Cref + i * ldr;
        double *s = Sabs ? Sabs + i * lds : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (s)
            for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)(transA ? A[k * lda + i] : A[i * lda + k]);
            for (int64_t j = 0; j < N; ++j) {
                const double b = (double)(transB ? B[j * ldb + k] : B[k * ldb + j]);
                const double prod = a * b;
                c[j] += prod;
                if (s) s[j] += fabs(prod);
            }
        }
        for (int64_t j = 0; j < N; ++j) {
            const double c0 = beta != 0.0 ? (double)C0[i * ldc0 + j] : 0.0;
            c[j] = alpha * c[j] + beta * c0;
            if (s) s[j] = fabs(alpha) * s[j] + fabs(beta) * fabs(c0);
        }
    }
    return ORACLE_OK;
}

/*
 * Selected entries of the general form, for products too large to compute
 * whole: entry e is (I[e], J[e]) of alpha op(A) op(B) + beta C0, with the same
 * ascending-k double sum, the same final combination and the same scale as
 * oracle_sgemm_ex_f64, so each entry equals that routine's bit for bit.
 */
int oracle_entries_ex_f64(int transA, int transB, int64_t M, int64_t N, int64_t K,
                          double alpha, const float *A, int64_t lda, const float *B,
                          int64_t ldb, double beta, const float *C0, int64_t ldc0, int64_t n,
                          const int64_t *I, const int64_t *J, double *cref, double *sabs)
{
    const int64_t acols = transA ? M : K, bcols = transB ? K : N;
    if (M < 0 || N < 0 || K < 0 || n < 0) return ORACLE_BAD_ARG;
    if (lda < (acols > 1 ? acols : 1) || ldb < (bcols > 1 ? bcols : 1)) return ORACLE_BAD_ARG;
    if (beta != 0.0 && ldc0 < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (n == 0) return ORACLE_OK;
    if (!I || !J || !cref || (K > 0 && (!A || !B)) || (beta != 0.0 && !C0)) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e)
        if (I[e] < 0 || I[e] >= M || J[e] < 0 || J[e] >= N) return ORACLE_BAD_ARG;
    for (int64_t e = 0; e < n; ++e) {
        const int64_t i = I[e], j = J[e];
        double c = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)(transA ? A[k * lda + i] : A[i * lda + k]);
            const double b = (double)(transB ? B[j * ldb + k] : B[k * ldb + j]);
            const double prod = a * b;
            c += prod;
            sa += fabs(prod);
        }
        const double c0 = beta != 0.0 ? (double)C0[i * ldc0 + j] : 0.0;
        cref[e] = alpha * c + beta * c0;
        if (sabs) sabs[e] = fabs(alpha) * sa + fabs(beta) * fabs(c0);
    }
    return ORACLE_OK;
}

/*
 * Vector addition C[i] = A[i] + B[i], i = 0 .. n-1, in single precision
 * [blog "【infra之路】03_动手写 CUDA Kernel", 实验 1 (experiment 1), the
 * vector-addition kernel: one element per thread, one add].  The result is
 * the correctly rounded (round-to-nearest-even) float sum: the sum is formed
 * in double and rounded once to float, and since double carries more than
 * 2 * 24 + 2 significand bits, rounding first to double and then to float
 * gives the same float as rounding the exact sum directly (the classical
 * double-rounding result for +, -, x, / and square root).  Returns
 * ORACLE_BAD_ARG for n < 0 or a null pointer with n > 0.
 */
int oracle_vector_add(int64_t n, const float *A, const float *B, float *C)
{
    if (n < 0 || (n > 0 && (!A || !B || !C)))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        C[i] = (float)((double)A[i] + (double)B[i]);
    return ORACLE_OK;
}

/*
 * Three-way split of a float into bfloat16 pieces, x = x0 + x1 + x2.  The
 * article "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式" names tensor
 * (matrix) cores as the next step (its closing summary, and the note under
 * its performance table) but gives no method; the reading taken here is the
 * usual one for carrying single precision through low-precision matrix
 * cores: split each operand into pieces the cores take exactly.  bfloat16
 * keeps the float exponent and 8 significant bits.  Each piece is the value
 * with 8 significant bits nearest to what is left, ties to even:
 *   x0 = rn8(x),  x1 = rn8(x - x0),  x2 = rn8(x - x0 - x1).
 * rn8 is written from its definition: x = f * 2^e with 1/2 <= |f| < 1, and
 * the result is nearbyint(f * 2^8) * 2^(e - 8) (nearbyint rounds to nearest
 * even in the default rounding mode).  For 2^-100 <= |x| <= 3.38e38 the
 * three pieces are normal bfloat16 values and their sum is x exactly; that is
 * the range the split is specified for.  Outputs are the bfloat16 bit
 * patterns (the high 16 bits of each piece as a float).  Returns
 * ORACLE_BAD_ARG for n < 0 or a null pointer with n > 0.
 */
static double rn8(double x)
{
    if (x == 0.0 || !isfinite(x))
        return x;
    int e;
    const double f = frexp(x, &e);
    return ldexp(nearbyint(ldexp(f, 8)), e - 8);
}

static uint16_t bf16_bits(double v)
{
    const float f = (float)v;  /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

int oracle_split_bf16x3(int64_t n, const float *x, uint16_t *p0, uint16_t *p1, uint16_t *p2)
{
    if (n < 0 || (n > 0 && (!x || !p0 || !p1 || !p2)))
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) {
        const double v = (double)x[i];
        const double x0 = rn8(v);
        const double x1 = rn8(v - x0);      /* v - x0 is exact in double */
        const double x2 = rn8(v - x0 - x1);
        p0[i] = bf16_bits(x0);
        p1[i] = bf16_bits(x1);
        p2[i] = bf16_bits(x2);
    }
    return ORACLE_OK;
}

/* Threads OpenMP would use by default; 1 when built without OpenMP. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
