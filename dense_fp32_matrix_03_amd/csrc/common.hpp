// common.hpp -- shared device helpers for the gfx950 single-precision kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;  // CDNA wavefront width

// v_mfma_f32_32x32x2_f32: D(32x32) = A(32x2) B(2x32) + C, one wave.
// Lane l supplies a = A(l % 32, l / 32) and b = B(l / 32, l % 32); register
// j of lane l holds D(8*(j/4) + 4*(l/32) + j%4, l % 32).
__device__ __forceinline__ f32x16 mfma32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4_f32: D(16x16) = A(16x4) B(4x16) + C, one wave.
// Lane l supplies a = A(l % 16, l / 16) and b = B(l / 16, l % 16); register
// j of lane l holds D(4*(l/16) + j, l % 16).
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row of register j of lane l in a 32x32 accumulator (column is l % 32).
__device__ __forceinline__ int acc32_row(int lane, int j) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

// Work-group id -> position in the launch order, grouping the work-groups that
// one XCD receives.  The dispatcher hands consecutive work-group ids to the
// 8 XCDs round robin, so id w runs on XCD w % 8.  Renumbering makes the ids
// that share an XCD (and so its L2) consecutive, so that the tile raster
// below gives each XCD a compact patch of C whose A rows and B columns it
// re-reads from its own L2.
__device__ __forceinline__ int xcd_contiguous_id(int w, int nwg) {
  constexpr unsigned kXcds = 8;
  const unsigned q = (unsigned)nwg / kXcds, r = (unsigned)nwg % kXcds;
  const unsigned x = (unsigned)w % kXcds, local = (unsigned)w / kXcds;
  return (int)(x * q + (x < r ? x : r) + local);
}

// Division by a divisor that is fixed for a launch, as one multiply and one
// shift (T. Granlund and P. L. Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, Theorem 4.2 with N = 31): for
// 1 <= d < 2^31, with l = ceil(log2 d) and m = ceil(2^(31+l) / d), which
// fits in 32 bits, floor(n / d) = floor(n m / 2^(31+l)) for every
// 0 <= n < 2^31.  The work-group -> tile maps divide by such divisors, built
// on the host, so a work-group spends a few scalar instructions before its
// first load instead of a reciprocal sequence per division.
struct FastDiv {
  unsigned m;
  int shift;
  __host__ __device__ __forceinline__ int operator()(int n) const {
    return (int)(((unsigned long long)(unsigned)n * m) >> shift);
  }
};

inline FastDiv make_fast_div(int d) {  // host side; 1 <= d < 2^31
  int l = 0;
  while ((1LL << l) < d) ++l;
  const unsigned long long p = 1ULL << (31 + l), dd = (unsigned long long)d;
  return FastDiv{(unsigned)((p + dd - 1) / dd), 31 + l};
}

// Launch position -> (product of the batch, tile row, tile column).  Tiles
// follow a grouped raster: groups of `group_m` tile rows, walked column by
// column inside a group, so work-groups that run together share both A row
// panels and B column panels.  Built once per launch (make_tile_map).
struct TileMap {
  int tiles_m, tiles_n, group_m;
  FastDiv by_tiles;        // tiles_m tiles_n: which product of the batch
  FastDiv by_group_tiles;  // group_m tiles_n: which group of tile rows
  FastDiv by_group_m;      // the rows of a full group
  FastDiv by_last_rows;    // the rows of a last, partial group
  __host__ __device__ __forceinline__ void tile(int id, int &bidx, int &tm, int &tn) const {
    bidx = by_tiles(id);
    const int t = id - bidx * (tiles_m * tiles_n);
    const int g = by_group_tiles(t);
    const int first = g * group_m;
    const int in = t - g * (group_m * tiles_n);
    const bool partial = first + group_m > tiles_m;
    const int rows = partial ? tiles_m - first : group_m;
    tn = partial ? by_last_rows(in) : by_group_m(in);
    tm = first + (in - tn * rows);
  }
};

inline TileMap make_tile_map(int tiles_m, int tiles_n, int group_m) {  // host side
  const int last = tiles_m % group_m;
  return TileMap{tiles_m,
                 tiles_n,
                 group_m,
                 make_fast_div(tiles_m * tiles_n),
                 make_fast_div(group_m * tiles_n),
                 make_fast_div(group_m),
                 make_fast_div(last ? last : group_m)};
}

}  // namespace sgemm

namespace sgemm {

// Arguments of one product, as the kernels see them.  Sizes are below 2^31
// (checked on the host); offsets into the operands are formed in 64 bits.
struct GemmArgs {
  int M, N, K;
  const float *A;
  long lda;
  const float *B;
  long ldb;
  float *C;
  long ldc;
  // The general form: C = alpha * op(A) op(B) + beta * C over `batch`
  // products whose operands start strideA / strideB / strideC floats apart.
  // The plain product keeps these defaults.
  float alpha = 1.f, beta = 0.f;
  long strideA = 0, strideB = 0, strideC = 0;
  int batch = 1;
  // Phase timestamps (the diagnostic instantiation only): 8 per work-group.
  unsigned long long *phases = nullptr;
};

// Register-staged fetch of a ROWS x COLS window (COLS a multiple of 4) of a
// row-major matrix, one 4-float chunk at a time.  Thread `tid` of NT owns the
// chunks q = tid + i*NT, i < CH: row q / (COLS/4) of the window, columns
// 4*(q % (COLS/4)) .. +3.  Elements at or beyond (rlim, clim) read as zero,
// which is how ragged edges are zero-filled (textbook chapter "4. 矩阵乘法性能
// 优化", section 三, boundary handling).  VEC selects one 128-bit load per
// chunk; it needs a 16-byte aligned base, ld % 4 == 0 and clim % 4 == 0, so
// that a chunk is either wholly inside or wholly outside.
template <int ROWS, int COLS, int NT, bool VEC>
struct SliceFetch {
  static constexpr int CPR = COLS / 4;           // chunks per window row
  static constexpr int CH = ROWS * CPR / NT;     // chunks per thread
  static constexpr int RSTEP = NT / CPR;         // rows between a thread's chunks
  static_assert(CH * NT == ROWS * CPR, "window must split evenly over the threads");
  static_assert(NT % CPR == 0, "threads must cover whole window rows");

  const float *p;  // first element of chunk 0
  long ld;
  int r, c;        // matrix row and column of chunk 0's first element
  f32x4 v[CH];

  __device__ __forceinline__ void init(const float *X, long ld_, int r0, int c0, int tid) {
    ld = ld_;
    r = r0 + tid / CPR;
    c = c0 + (tid % CPR) * 4;
    p = X + (long)r * ld + c;
  }

  __device__ __forceinline__ void load(int rlim, int clim) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ri = r + i * RSTEP;
      const float *pi = p + (long)(i * RSTEP) * ld;
      if constexpr (VEC) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        if (ri < rlim && c < clim) t = *reinterpret_cast<const f32x4 *>(pi);
        v[i] = t;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[i][e] = (ri < rlim && c + e < clim) ? pi[e] : 0.f;
      }
    }
  }

  __device__ __forceinline__ void advance(int dr, int dc) {
    r += dr;
    c += dc;
    p += (long)dr * ld + dc;
  }

  // Window coordinates of chunk i (row, first column) for the LDS store.
  __device__ __forceinline__ static int wrow(int tid, int i) { return tid / CPR + i * RSTEP; }
  __device__ __forceinline__ static int wcol(int tid) { return (tid % CPR) * 4; }
};

}  // namespace sgemm
