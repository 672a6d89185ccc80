// dispatch.hpp -- host-side launchers of the kernels (C++ linkage, internal).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sgemm {

// Block tiles of the matrix-core kernels (mfma_configs.hpp gives the wave
// grids of the buffer-to-LDS kernel): 256 x 256, 128 x 128, 64 x 96 (K split
// over two sets of six waves), 64 x 64, 32 x 64 (two k sets) and 32 x 32
// (four k sets); and 16 x 16, the small-product kernel (mfma_small.hip: four
// k sets of one wave, operands loaded straight into registers).
enum class MfmaTile { T256, T128, T64x96, T64, T32x64, T32, T16 };

// A tile and its form.  long_k selects 64-float K slices; ksplit (64 x 64
// only) runs the tile with two k sets of four waves.
//  - The four-wave tiles (32 x 64, 32 x 32) take 64-float slices when all
//    their work-groups fit one round on the compute units: no second
//    work-group per CU hides the per-slice barrier, and half as many slices
//    halve its cost.
//  - The 64 x 64 tile takes two k sets (8 waves) when its work-groups fit
//    one round and K >= 512 (1024^3: 18.95 -> 18.4 us), with 64-float slices
//    from K >= 1280.  Each XCD's 32 work-groups read 8 tile rows of A and 4
//    tile columns of B, 3 KiB per k; up to K = 1280 that fits the XCD's 4 MB
//    L2 and back-to-back calls find their operands there, beyond it the
//    operands come from farther away, and a 32-float slice (0.43 us of
//    matrix work per SIMD at 1024^2) does not cover that latency: 1024 x
//    1024 x 1408 takes 28.8 us on 32-float slices against 24.0 on 64-float
//    ones, 1024^2 x 1536 31.5 against 26.1, while 1024^2 x 1152 and 1280 take
//    the same time on both and 1024^3 is 1.5 % faster on 32-float slices.
//    Otherwise the four-wave form: with several work-groups per CU, or few
//    K slices, the eight-wave form loses (1024 products of 64^3: 9.8 against
//    16.2 us; 3072 x 3072 x 1024: 136.8 against 139.6 us).
//  - The 64 x 96 tile has one form: 32-float slices, two k sets of six waves.
//  - The 16 x 16 tile has no K slices; where a variant runs the
//    buffer-to-LDS kernel instead, it takes the 32 x 32 tile's form.
struct TileChoice {
  MfmaTile tile;
  bool long_k;
  bool ksplit;
};

// Which matrix-core kernel:
//  Auto      the 16 x 16 tile's small-product kernel; else buffer-to-LDS
//            loads (16 bytes per lane where va / vb, else 4), or
//            register-staged loads when a slice's offsets do not fit a
//            buffer descriptor (a leading dimension near 2^29 or more);
//  Staged    register-staged loads always (the 16 x 16 tile takes 64 x 64);
//  Unpadded  buffer-to-LDS without the LDS anti-conflict layout (no A
//            swizzle), to measure what that layout buys (the 16 x 16 tile
//            takes 32 x 32);
//  Serial    the race-triage schedule of the buffer-to-LDS kernel
//            (hipErrorInvalidValue where Auto would fall back to the
//            register-staged kernel); the small-product kernel stages
//            nothing through LDS and runs unchanged.
enum class MfmaPath { Auto, Staged, Unpadded, Serial };

// The tile for `batch` products of M x N x K on `cus` compute units: the
// buffer-to-LDS tile that wastes the least matrix-core time to partly filled
// rounds of work-groups and to tile area outside C, preferring the larger
// tile when two come within 3% of each other, and the 64 x 96 tile only
// where its work-groups fit one round on the compute units -- unless
// small_product() holds and either the 16 x 16 tiles read at most 56 KiB per
// compute unit or that best tile keeps under half of the matrix-core time on
// C: then the 16 x 16 tile.
TileChoice choose_mfma_tile(long M, long N, long K, int cus, long batch = 1);

// Whether the 16 x 16 small-product kernel serves the product: K <= 1024,
// at most 8 of its tiles per compute unit, and its tiles' operand reads
// (128 K bytes per tile, each wave loading its own) at most 128 KiB per
// compute unit.
bool small_product(long M, long N, long K, int cus, long batch = 1);

// `tile` with the K-slice length choose_mfma_tile would give it.
TileChoice with_slice_rule(MfmaTile tile, long M, long N, long K, int cus, long batch = 1);

// What a tile choice launches for the plain layout (wide: both operands take
// 16-byte loads): block tile bm x bn, K slice bk (for the 16 x 16 tile, the K
// one pass of its four waves covers) and the number of k sets.
struct TileGeometry {
  int bm, bn, bk, ksets;
};
TileGeometry tile_geometry(TileChoice tile, bool wide, long K);

// Which operands take 16-byte loads.  a16 / b16: A / B qualify for the
// small-product and register-staged kernels (16-byte aligned, leading
// dimension and stored width multiples of 4).  a_dma / b_dma: A / B qualify
// for the buffer-to-LDS kernel, which needs only dword alignment, and a
// stored width that is a multiple of 4 where its 16-byte chunks run along m
// or n (A stored transposed, B as given); all false forces 4-byte loads.
struct LoadWidths {
  bool a16 = false, b16 = false, a_dma = false, b_dma = false;
};

// Matrix-core product.
hipError_t launch_mfma(TileChoice tile, MfmaPath path, const GemmArgs &p, LoadWidths w,
                       hipStream_t stream);

// General product C = alpha op(A) op(B) + beta C over p.batch products on
// the buffer-to-LDS kernel (ta / tb: A / B stored transposed).  Returns
// hipErrorInvalidValue if a slice's offsets do not fit a buffer descriptor.
hipError_t launch_mfma_general(TileChoice tile, const GemmArgs &p, bool ta, bool tb, LoadWidths w,
                               hipStream_t stream);

// sgemm_run's computation of the plain product with phase timestamps in
// p.phases (8 per work-group); *workgroups receives the launch's work-group
// count.  With p.phases null nothing is launched.  hipErrorInvalidValue if a
// slice's offsets do not fit a buffer descriptor.
hipError_t launch_mfma_phases(TileChoice tile, const GemmArgs &p, LoadWidths w, long *workgroups,
                              hipStream_t stream);

// Small-product kernel (mfma_small.hip) over p.batch products: 16 x 16 tiles,
// four k sets of one wave, operands loaded straight into registers (ta / tb:
// A / B stored transposed; va / vb: the operand qualifies for 16-byte loads).
// Any K (in chunks of 1024 beyond that).
hipError_t launch_small(const GemmArgs &p, bool ta, bool tb, bool va, bool vb,
                        hipStream_t stream);
// The same for the plain layout with phase timestamps in p.phases.
hipError_t launch_small_phases(const GemmArgs &p, bool va, hipStream_t stream);
// Work-groups of the small-product kernel for `batch` products of M x N.
long small_workgroups(long M, long N, long batch);

// Register-staged kernel (mfma_gemm.hpp) on a 256, 128 or 64 tile (others
// take 64); padded = false drops its A row padding.
hipError_t launch_staged(MfmaTile tile, bool padded, const GemmArgs &p, bool va, bool vb,
                         hipStream_t stream);

// C = beta * C over p.batch products (zeros when beta == 0; C not read).
hipError_t launch_scale(const GemmArgs &p, hipStream_t stream);

// One-instruction lane-layout probe (which: 0 = 32x32x2, 1 = 16x16x4).
hipError_t launch_mfma_probe(int which, const float *A, const float *B, float *C,
                             hipStream_t stream);

// Vector-FMA progression: 0 naive, 1 LDS-tiled, 2 register-tiled,
// 3 register-tiled with a double-buffered LDS pipeline.
hipError_t launch_valu(int rung, const GemmArgs &p, bool va, bool vb, hipStream_t stream);

// ---- single precision through the bfloat16 matrix cores (bf16x3.hip)
// Operands split into three bfloat16 planes with k contiguous, K padded with
// zeros to Kp (a multiple of 32): a = [3][M][Kp], b = [3][N][Kp].
struct Bf16x3Args {
  int M, N;
  long Kp;
  const unsigned short *a, *b;
  long plane_a, plane_b;  // bfloat16 per plane: M * Kp, N * Kp
  float *C;
  long ldc;
  float alpha = 1.f, beta = 0.f;  // C = alpha (product) + beta C; C read only if beta != 0
};

// Split op(A) (M x K) into wa = [3][M][Kp] and op(B) (K x N) into wb =
// [3][N][Kp] bfloat16 planes, in one launch; ta / tb: A / B stored
// transposed (A as K x M with leading dimension lda, B as N x K).
hipError_t launch_split(bool ta, bool tb, const float *A, long lda, const float *B, long ldb,
                        int M, int N, int K, int Kp, void *wa, void *wb, hipStream_t stream);

// C = alpha (sum of the six piece products over the planes) + beta C, on a
// tile chosen for `cus` compute units.  hipErrorInvalidValue if a slice's
// offsets do not fit a buffer descriptor.
hipError_t launch_bf16x3_gemm(const Bf16x3Args &p, int cus, hipStream_t stream);

// One-instruction probe of the bfloat16 32x32x16 matrix instruction.
hipError_t launch_bf16_probe(const float *A, const float *B, float *C, hipStream_t stream);

// Register-only matrix-core loop on every CU (which: 0 = FP32 32x32x2,
// 1 = bfloat16 32x32x16); *flops receives the launch's flop count.  `out`
// holds mfma_ceiling_outputs(cus) floats.
long mfma_ceiling_outputs(int cus);
hipError_t launch_mfma_ceiling(int which, int iters, float *out, int cus, double *flops,
                               hipStream_t stream);

// C[i] = A[i] + B[i], i < n (n >= 1).
hipError_t launch_vector_add(long n, const float *A, const float *B, float *C,
                             hipStream_t stream);

}  // namespace sgemm
