/*
 * sgemm.h -- C interface of libsgemm, a single-precision matrix product for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  C = A x B for row-major single-precision matrices, where A
 * is M x K, B is K x N and C is M x N, and entry (i, j) of C is the sum over
 * k of A(i,k) * B(k,j).  Definition: article "硬件加速原理：CUDA核函数优化矩阵
 * 乘法的内存访问模式", section "矩阵乘法的计算特性" (the summation formula), and
 * the opening paragraph of the textbook chapter "4. 矩阵乘法性能优化".  The
 * pages' kernels overwrite C with the sum and never read it; so do
 * sgemm_run and sgemm_run_variant.  sgemm_run_ex and sgemm_run_strided_batched
 * (below) add the general form alpha * op(A) op(B) + beta * C.
 *
 * Layout.  Element (i, k) of A is A[i*lda + k]; element (k, j) of B is
 * B[k*ldb + j]; element (i, j) of C is C[i*ldc + j] (the row-major indexing
 * of the blog "【infra之路】03_动手写 CUDA Kernel", v1 Naive, generalised to
 * leading dimensions).  Requirements: lda >= max(1, K), ldb >= max(1, N),
 * ldc >= max(1, N).  Columns j in [N, ldc) of C are never written; columns
 * beyond K of A and beyond N of B are never read into the result.
 *
 * Numerics.  Products and sums are single precision with fused multiply-add
 * (the matrix cores fuse); the order of summation is fixed for a given call
 * shape, so repeated calls give identical bits.  The accuracy contract is
 * |C(i,j) - exact| <= 1e-5 * sum_k |A(i,k) B(k,j)| + 1e-6 for finite inputs.
 * NaN or infinite inputs are outside the contract.
 *
 * Pointers and ownership.  A, B and C are device pointers owned by the
 * caller; the library allocates no memory per call and keeps no pointer
 * after a call returns.  C must not overlap A or B.  Any 4-byte alignment is
 * accepted.  The matrix-core path fetches an operand in 16-byte chunks from
 * any 4-byte aligned address wherever no chunk would cross the edge of the
 * operand (the stored width a multiple of 4 where the chunks run along m or
 * n); the other kernels need 16-byte alignment and leading dimensions and
 * widths that are multiples of 4 for 16-byte loads.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 * stream of the current device).  Calls are asynchronous: they return once
 * the work is enqueued on the current device; a fault in the kernel shows up
 * at the caller's next synchronisation with that stream.
 *
 * Errors.  Every call returns SGEMM_OK (0) or a negative status; nothing is
 * enqueued when a status other than SGEMM_OK is returned, except
 * SGEMM_ERR_LAUNCH, which reports that the runtime rejected a launch.
 * Argument errors (SGEMM_ERR_INVALID_VALUE, SGEMM_ERR_TOO_LARGE) are found
 * before the library or the HIP runtime is consulted, so they are reported
 * even before sgemm_create.  sgemm_status_string() names each status.
 * Limits (SGEMM_ERR_TOO_LARGE): M, N, K and batch below 2^31, and one launch
 * below 2^32 work-items.  sgemm_run and the general form take any product
 * with at most 2^24 blocks of 64 x 64 (counting every product of a batch)
 * and pick a tile whose launch fits; the forced tiles need 512 work-items
 * per 64 x 64 block (SGEMM_VARIANT_MFMA_64), 768 per 64 x 96 block
 * (SGEMM_VARIANT_MFMA_64X96) or 256 per 32 x 64 (SGEMM_VARIANT_MFMA_32X64),
 * 32 x 32 (SGEMM_VARIANT_MFMA_32) or 16 x 16 block (SGEMM_VARIANT_MFMA_16),
 * the vector-FMA variants 256 per 16 x 16 block.
 *
 * Threads.  sgemm_create / sgemm_destroy are serialised internally;
 * sgemm_run may be called from any thread once sgemm_create has succeeded.
 */
#ifndef SGEMM_H_
#define SGEMM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_OK 0
#define SGEMM_ERR_INVALID_VALUE (-1)    /* negative size, short ld, null pointer, bad variant */
#define SGEMM_ERR_NOT_INITIALIZED (-2)  /* sgemm_run before sgemm_create */
#define SGEMM_ERR_UNSUPPORTED_DEVICE (-3) /* current device is not gfx950 */
#define SGEMM_ERR_HIP (-4)              /* a HIP runtime query failed */
#define SGEMM_ERR_LAUNCH (-5)           /* the runtime rejected a kernel launch */
#define SGEMM_ERR_TOO_LARGE (-6)        /* a size is past the library's limits */

/*
 * Kernel variants for sgemm_run_variant.  The first four are the pages'
 * progression on vector FMA units -- one thread per output (blog v1 Naive;
 * the article's basic kernel, section "矩陣乘法基礎與CUDA實現原理"), LDS
 * tiling (blog v2 Shared Memory Tiled; chapter section 三), register tiling
 * with 8x8 outputs per thread over 128x128x16 blocks (chapter sections 一
 * and 二), and that with a double-buffered LDS pipeline (chapter section
 * 四).  SGEMM_VARIANT_MFMA is the matrix-core path that sgemm_run uses:
 * operand slices reach LDS by buffer-to-LDS loads of 16 bytes per lane
 * from any 4-byte aligned address, and of 4 bytes in the partial last K
 * slice when K % 4 != 0 and, on the 64 x 96 tile, for operands that are not
 * 16-byte aligned with a leading dimension and width that are multiples of
 * 4 or once a ragged K reaches 960; only an operand whose leading
 * dimension puts one slice beyond 2 GiB is fetched through registers
 * instead.  sgemm_run
 * picks the block tile (256 x 256, 128 x 128, 64 x 96, 64 x 64, 32 x 64 or
 * 32 x 32) that loses the least matrix-core time to partly filled rounds of
 * work-groups and to tile area outside C, the larger one when two come
 * within 3%; the 64 x 96 tile only where its work-groups fit one round on
 * the compute units.  A product with K <= 1024, at most 8 tiles of 16 x 16 per
 * compute unit and at most 128 KiB of operand reads per compute unit on
 * those tiles (128 K bytes per tile) takes the 16 x 16 tile instead when
 * those reads stay within 48 KiB per compute unit or the best of the other
 * tiles would spend under half of the matrix-core time on C.  The
 * _MFMA_<n> variants force a tile (with the same rule for its form): the
 * 64 x 64 tile runs four waves, or two sets of four when its work-groups fit
 * one round on the compute units and K >= 512; the 64 x 96 tile two sets of
 * six waves (one work-group fills a CU), the 32 x 64 tile two sets of two
 * waves and the 32 x 32 tile four single waves, each set summing its share
 * of every K slice; the 16 x 16 tile (the 16x16x4 matrix instruction)
 * four single waves that load their share of K straight from global memory
 * into registers, with no LDS staging.  The sets' partial sums are added in
 * a fixed order.  SGEMM_VARIANT_MFMA_STAGED always fetches through
 * registers, SGEMM_VARIANT_MFMA_UNPADDED drops the LDS anti-conflict
 * layout (the chapter's padding, section 三), and SGEMM_VARIANT_MFMA_DWORD
 * fetches both operands 4 bytes per lane even where 16-byte loads are
 * allowed (the article's coalescing section, "内存合并访问原理": the width
 * of each lane's access sets how many bytes one wave instruction moves):
 * all three exist to measure what those steps are worth.
 * SGEMM_VARIANT_MFMA_SERIAL is a race-triage form of SGEMM_VARIANT_MFMA: the
 * same tile, loads and matrix-core sequence, hence the same bits, but every
 * K slice is computed with no load in flight and with extra workgroup
 * barriers (after each slice's loads are issued and before each group of LDS
 * reads; the chapter's section 四 explains the two barriers a pipelined
 * slice needs).  A result that differs between the two points to a missing
 * wait or barrier, one that does not to the arithmetic.  It returns
 * SGEMM_ERR_TOO_LARGE where sgemm_run would fetch through registers.  The
 * 16 x 16 tile stages nothing through LDS and runs unchanged; the
 * register-staged and unswizzled variants run it as 64 x 64 and 32 x 32.
 */
#define SGEMM_VARIANT_NAIVE 0
#define SGEMM_VARIANT_LDS 1
#define SGEMM_VARIANT_REG 2
#define SGEMM_VARIANT_DBUF 3
#define SGEMM_VARIANT_MFMA 4
#define SGEMM_VARIANT_MFMA_256 5
#define SGEMM_VARIANT_MFMA_128 6
#define SGEMM_VARIANT_MFMA_64 7
#define SGEMM_VARIANT_MFMA_STAGED 8
#define SGEMM_VARIANT_MFMA_UNPADDED 9
#define SGEMM_VARIANT_MFMA_32 10
#define SGEMM_VARIANT_MFMA_DWORD 11
#define SGEMM_VARIANT_MFMA_32X64 12
#define SGEMM_VARIANT_MFMA_SERIAL 13
#define SGEMM_VARIANT_MFMA_16 14
#define SGEMM_VARIANT_MFMA_64X96 15
#define SGEMM_NUM_VARIANTS 16

/*
 * Initialise the library for the current device: checks that it is gfx950
 * and caches its compute-unit count.  Reference counted; each successful
 * call must be matched by sgemm_destroy.  Returns SGEMM_OK,
 * SGEMM_ERR_UNSUPPORTED_DEVICE or SGEMM_ERR_HIP.
 */
int sgemm_create(void);

/* Drop one reference taken by sgemm_create.  SGEMM_ERR_NOT_INITIALIZED if none. */
int sgemm_destroy(void);

/*
 * C = A x B on `stream` (see the layout and numerics above).  M == 0 or
 * N == 0 is a successful no-op; K == 0 writes zeros to the M x N block of C
 * (the empty sum).  A and B may be NULL when M*N*K == 0; C may be NULL when
 * M*N == 0.
 */
int sgemm_run(int64_t M, int64_t N, int64_t K,
              const float *A, int64_t lda,
              const float *B, int64_t ldb,
              float *C, int64_t ldc, void *stream);

/*
 * Same contract as sgemm_run, computed by kernel `variant`
 * (SGEMM_VARIANT_*).  Every variant meets the same accuracy contract.
 * SGEMM_ERR_INVALID_VALUE for an unknown variant.
 */
int sgemm_run_variant(int variant, int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      float *C, int64_t ldc, void *stream);

/*
 * The general form: C = alpha * op(A) op(B) + beta * C, the plain product
 * extended by the two steps around it.  The article "硬件加速原理：CUDA核函数
 * 优化矩阵乘法的内存访问模式" (section "访问模式对比") contrasts row- and
 * column-major operands; transposed operands are how a row-major interface
 * takes column-major data.
 *
 * op(A) is M x K: A itself (transA == 0, stored M x K, lda >= max(1, K)) or
 * the transpose of a stored K x M matrix (transA == 1, lda >= max(1, M),
 * op(A)(i,k) = A[k*lda + i]).  op(B) is K x N: B itself (transB == 0, stored
 * K x N, ldb >= max(1, N)) or the transpose of a stored N x K matrix
 * (transB == 1, ldb >= max(1, K), op(B)(k,j) = B[j*ldb + k]).  C is M x N,
 * ldc >= max(1, N).  When beta == 0, C is only written (NaN or Inf in it do
 * not propagate); when alpha == 0 or K == 0, A and B are not read and
 * C = beta * C.  Products are summed in single precision as in sgemm_run;
 * the result is alpha * sum + beta * C, rounded once after beta * C.
 * Returns SGEMM_ERR_TOO_LARGE, besides the cases of sgemm_run, when a
 * leading dimension is so large that one K slice spans 2 GiB.
 */
int sgemm_run_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                 const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                 float *C, int64_t ldc, void *stream);

/*
 * `batch` independent general products on one stream: product b uses
 * A + b*strideA, B + b*strideB and C + b*strideC (strides in floats,
 * >= 0; a stride of 0 shares that operand).  The C matrices of different
 * products must not overlap: with batch > 1, strideC < (M - 1) * ldc + N is
 * SGEMM_ERR_INVALID_VALUE.  Many small products in one launch fill the
 * device where one alone cannot; batched matrix work is the subject that the
 * address of the textbook chapter "4. 矩阵乘法性能优化" names.  batch == 0 is
 * a no-op.
 */
int sgemm_run_strided_batched(int transA, int transB, int64_t M, int64_t N, int64_t K,
                              float alpha, const float *A, int64_t lda, int64_t strideA,
                              const float *B, int64_t ldb, int64_t strideB, float beta,
                              float *C, int64_t ldc, int64_t strideC, int64_t batch,
                              void *stream);

/*
 * Matrix-core layout probe: one wave multiplies a 32 x 2 block of A by a
 * 2 x 32 block of B (which = 0, v_mfma_f32_32x32x2_f32), a 16 x 4 block by
 * a 4 x 16 block (which = 1, v_mfma_f32_16x16x4_f32), or a 32 x 16 block by
 * a 16 x 32 block in bfloat16 (which = 2, v_mfma_f32_32x32x16_bf16; the
 * high 16 bits of each float input are its bfloat16 value), with A and B
 * row-major and packed, and writes the 32 x 32 (or 16 x 16) product
 * row-major and packed to C.  It exercises the operand and accumulator lane
 * maps that the matrix-core kernels rely on.  SGEMM_ERR_INVALID_VALUE for
 * another `which` or a null pointer.
 */
int sgemm_mfma_probe(int which, const float *A, const float *B, float *C, void *stream);

/*
 * Matrix-core ceiling: a register-only loop of `iters` iterations over eight
 * independent accumulator chains per wave, four 256-thread work-groups per
 * compute unit, on every compute unit of the current device, with no memory
 * traffic; which = 0 times v_mfma_f32_32x32x2_f32, which = 1
 * v_mfma_f32_32x32x16_bf16.  It measures the rate the matrix cores attain,
 * against which a product kernel's rate is read beside the published peak.
 * `out` is a device buffer of out_len floats that receives one sum per
 * thread (at least 1024 per compute unit); *flops (host memory) receives the
 * launch's flop count.  SGEMM_ERR_INVALID_VALUE for another `which`,
 * iters < 1, a null pointer or a short `out`.
 */
int sgemm_mfma_ceiling(int which, int iters, float *out, int64_t out_len, double *flops,
                       void *stream);

/*
 * Diagnostic: sgemm_run's computation of C = A x B (the same tile choice,
 * kernel code and result bits, for operands that take the buffer-to-LDS
 * path) with timestamps that show where a call's time goes.  Thread 0 of
 * each work-group w records, in the device buffer `times`, times[8w + i] for
 *   i = 0  start of the work-group,
 *       1  its first K slice has landed in LDS (the first load's latency),
 *       2  its last slice is computed (the main loop),
 *       3  the partial sums of its k sets are added (tiles that split K),
 *       4  its stores of C are complete,
 * on the device's constant reference clock (s_memrealtime, 100 MHz on
 * MI355X), its shader clock (s_memtime, in cycles) at the start and at the
 * end in times[8w + 5] and times[8w + 6], and its tile in times[8w + 7]:
 * BM | BN << 16 | BK << 32 | KSPLIT << 48 (block rows and columns, K-slice
 * length, k sets).  Waiting for the stores before
 * the last timestamp is the only difference from sgemm_run's kernel, which
 * leaves that wait to the end of the dispatch.  These are the pipeline
 * stages of the textbook chapter "4. 矩阵乘法性能优化" (sections 一 to 四) and
 * the measurement its section 五 asks for.
 *
 * *workgroups (host) receives the work-group count; with times == NULL
 * nothing is launched (a size query).  M, N and K must be at least 1
 * (SGEMM_ERR_INVALID_VALUE); times_len < 8 * *workgroups is
 * SGEMM_ERR_INVALID_VALUE; SGEMM_ERR_TOO_LARGE where sgemm_run would fetch
 * through registers (a leading dimension that puts one K slice beyond 2 GiB).
 * Other checks and statuses as for sgemm_run.
 */
int sgemm_phase_times(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, uint64_t *times,
                      int64_t times_len, int64_t *workgroups, void *stream);

/*
 * The matrix-core configuration that sgemm_run (batch = 1) and the general
 * form choose for `batch` products of M x N x K on a device with `cus`
 * compute units, for the plain layout with 16-byte loads on both operands
 * (the rule is described with the variants above).  Host logic only: no
 * device call, and no sgemm_create needed.  Writes the block tile
 * (*bm x *bn), the K slice *bk (for the 16 x 16 tile, the K that one pass
 * of its four waves covers) and the number of k sets *ksets (host memory).
 * SGEMM_ERR_INVALID_VALUE for M, N, K, batch or cus below 1 or a null
 * pointer; SGEMM_ERR_TOO_LARGE past sgemm_run's limits.
 */
int sgemm_tile_choice(int64_t M, int64_t N, int64_t K, int64_t batch, int cus, int *bm, int *bn,
                      int *bk, int *ksets);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char *sgemm_status_string(int status);

/* Static, NUL-terminated name of a variant, or NULL for an unknown one. */
const char *sgemm_variant_name(int variant);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H_ */
