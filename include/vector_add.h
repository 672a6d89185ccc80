/*
 * vector_add.h -- element-wise single-precision vector addition on MI355X
 * (gfx950), part of libsgemm.so.
 *
 * Operation.  C[i] = A[i] + B[i] for i = 0 .. n-1, each sum rounded to the
 * nearest float (ties to even) [blog "【infra之路】03_动手写 CUDA Kernel — 向量加法
 * 到矩阵乘法", 实验 1 (experiment 1), the vector-addition kernel].  The blog
 * times it over n = 2^24 floats and counts three arrays of n floats (A and B
 * read, C written) as its effective bandwidth; here it is the measured
 * streaming ceiling that the product kernels' memory traffic is compared to.
 *
 * Layout and ownership.  A, B and C are device pointers to n floats each,
 * owned by the caller; any alignment is accepted (16-byte aligned arrays take
 * 16-byte loads and stores).  C may be the same pointer as A or B; other
 * overlaps are undefined.  The call is asynchronous on `stream` (a
 * hipStream_t passed as void*, NULL for the null stream) and allocates
 * nothing.
 *
 * Status codes are those of sgemm.h.  Errors, checked in this order:
 * SGEMM_ERR_INVALID_VALUE for n < 0 or a null pointer with n > 0;
 * SGEMM_ERR_TOO_LARGE for n > 2^33; SGEMM_ERR_NOT_INITIALIZED before
 * sgemm_create; SGEMM_ERR_UNSUPPORTED_DEVICE / SGEMM_ERR_HIP from the device
 * check; SGEMM_ERR_LAUNCH if the runtime rejects the launch.  n == 0 is a
 * successful no-op.
 */
#ifndef VECTOR_ADD_H_
#define VECTOR_ADD_H_

#include <stdint.h>

#include "sgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

int vector_add(int64_t n, const float *A, const float *B, float *C, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* VECTOR_ADD_H_ */
