/*
 * sgemm_bf16x3.h -- the single-precision product C = A x B computed on the
 * bfloat16 matrix cores of MI355X (gfx950), part of libsgemm.so.
 *
 * Operation and accuracy.  The same product and the same contract as
 * sgemm_run (sgemm.h): row-major A (M x K), B (K x N), C (M x N) with leading
 * dimensions, entry (i, j) = sum over k of A(i,k) B(k,j) [article
 * "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式", section
 * "矩阵乘法的计算特性"], |C - exact| <= 1e-5 * sum_k |A(i,k) B(k,j)| + 1e-6.
 * The article names tensor (matrix) cores as the next step but gives no
 * method; here each operand value is split into three bfloat16 pieces,
 * x = x0 + x1 + x2 with each piece the nearest bfloat16 to what is left
 * (ties to even), and C accumulates, in single precision, the six piece
 * products a_i b_j with i + j <= 2.  The dropped products are below
 * 2^-23 |a b|.  This holds for operands with 2^-100 <= |x| <= 3.38e38 (or
 * x = 0); smaller magnitudes lose relative accuracy (absolutely below
 * 2^-100), larger ones overflow the first piece.  NaN and infinity are
 * outside the contract.  Integer-valued operands below 2^8 in magnitude are
 * exact in the first piece, so such products are exact while the sums stay
 * below 2^24.
 *
 * Workspace.  The caller supplies device memory of at least
 * sgemm_bf16x3_workspace_size(M, N, K) bytes, 16-byte aligned.  A call
 * writes the split operands there -- with Kp = K rounded up to a multiple
 * of 32: op(A) as three planes [3][M][Kp] of bfloat16 (k contiguous), then
 * op(B) transposed as [3][N][Kp], padding columns zero; the planes are the
 * same whichever way an operand is stored -- and reads them back in the
 * product.  The contents are only meaningful until the next call that
 * uses the same workspace; two calls in flight on different streams must not
 * share one.  The library allocates nothing.
 *
 * Everything else -- pointer ownership, streams, asynchrony, M == 0 / N == 0
 * / K == 0, status codes, the check order -- is as for sgemm_run.  Extra
 * errors: SGEMM_ERR_INVALID_VALUE for a null, misaligned or too small
 * workspace when M, N and K are all positive; SGEMM_ERR_TOO_LARGE for
 * K > 2^21 or (M + N) * Kp > 2^34.
 *
 * sgemm_run_bf16x3_ex is the general form of sgemm_run_ex (sgemm.h) on the
 * same split: C = alpha * op(A) op(B) + beta * C with the transposes, the
 * leading-dimension rules, the alpha == 0 / beta == 0 behaviour and the
 * rounding of alpha * sum + beta * C of sgemm_run_ex, and the accuracy
 * contract above for the sum.  The workspace is needed, and the workspace
 * errors and size limits apply, only when M, N and K are positive and
 * alpha != 0 (otherwise A, B and the workspace are not touched).
 * sgemm_run_bf16x3 is sgemm_run_bf16x3_ex(0, 0, M, N, K, 1, A, lda, B, ldb,
 * 0, C, ldc, ...).
 */
#ifndef SGEMM_BF16X3_H_
#define SGEMM_BF16X3_H_

#include <stdint.h>

#include "sgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes for an M x N x K call (0 when K == 0), or a negative
 * status: SGEMM_ERR_INVALID_VALUE for negative sizes, SGEMM_ERR_TOO_LARGE as
 * above. */
int64_t sgemm_bf16x3_workspace_size(int64_t M, int64_t N, int64_t K);

int sgemm_run_bf16x3(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float *C, int64_t ldc,
                     void *workspace, int64_t workspace_bytes, void *stream);

int sgemm_run_bf16x3_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                        float *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                        void *stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * call as sgemm_run_bf16x3_ex, without the workspace arguments.  The split
 * planes go to a buffer the library holds on each GPU it runs on
 * (SGEMM_BF16X3_NOALLOC_MAX_BYTES, 64 MiB, kept until the process ends and
 * set up by the runtime when this entry point is first called on that GPU);
 * the call itself allocates nothing and calls no allocating routine.
 *
 * Limit: a call whose workspace, sgemm_bf16x3_workspace_size(M, N, K),
 * exceeds SGEMM_BF16X3_NOALLOC_MAX_BYTES returns SGEMM_ERR_TOO_LARGE before
 * anything is enqueued (2048 x 2048 x 2048 needs 50.3 MB and fits; 4096^3
 * does not).  Every other status, check and result is exactly that of
 * sgemm_run_bf16x3_ex with a large enough workspace: the results are bit for
 * bit the same.  SGEMM_ERR_HIP if the buffer's device address cannot be
 * looked up.
 *
 * Every call on one GPU shares that GPU's buffer: calls that overlap on one
 * GPU (in flight together on different streams, or from different host
 * threads) race and must be ordered by the caller.  Each call rewrites
 * every byte of the buffer it reads, so nothing left by an earlier call
 * affects a later one.
 */
#define SGEMM_BF16X3_NOALLOC_MAX_BYTES (64ll << 20)

int sgemm_run_bf16x3_ex_noalloc(int transA, int transB, int64_t M, int64_t N, int64_t K,
                                float alpha, const float *A, int64_t lda, const float *B,
                                int64_t ldb, float beta, float *C, int64_t ldc, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_BF16X3_H_ */
