// bf16x3.hip -- the single-precision product C = A x B carried through the
// bfloat16 matrix cores of gfx950.
//
// The article "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式" names tensor
// (matrix) cores as the next step beyond its FP32 kernels.  On gfx950 the
// bfloat16 matrix instruction has 16 times the throughput of the FP32 one,
// but a bfloat16 keeps only 8 significant bits.  So each operand value is
// split into three bfloat16 pieces that sum to it exactly,
//   x = x0 + x1 + x2,  x0 = rn(x), x1 = rn(x - x0), x2 = x - x0 - x1
// (rn: nearest bfloat16, ties to even; |x1| <= 2^-8 |x|, |x2| <= 2^-16 |x|),
// and the product keeps the six piece products whose order adds up to at
// most 2:  a0 b0 + a0 b1 + a1 b0 + a0 b2 + a1 b1 + a2 b0.  The three dropped
// products are below 2^-23 |a b| together, under single-precision rounding;
// each piece product is exact in the FP32 accumulator.  Six bfloat16
// instructions cost 6/16 of one FP32 instruction.
//
// Two passes:
//  1. split: each operand is read once from HBM and written to the caller's
//     workspace as three bfloat16 planes with k contiguous, K padded with
//     zeros to Kp (a multiple of 32): op(A) as [3][M][Kp], op(B) transposed
//     as [3][N][Kp], whichever way each operand is stored.  Memory-bound,
//     like the vector add.
//  2. product: the buffer-to-LDS pipeline of the FP32 kernel (mfma_dma.hpp)
//     over the six planes, v_mfma_f32_32x32x16_bf16 on 32 x 32 blocks, and
//     the FP32 kernel's alpha / beta epilogue.
#include "common.hpp"
#include "dispatch.hpp"
#include "mfma_dma.hpp"

namespace sgemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16: D(32x32) = A(32x16) B(16x32) + C, one wave.
// Lane l supplies the 8 values A(l % 32, 8*(l/32) + e) and B(8*(l/32) + e,
// l % 32), e < 8; the accumulator layout is that of the FP32 32x32
// instruction (acc32_row).
__device__ __forceinline__ f32x16 mfma32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Split 8 floats into three 16-byte chunks of bfloat16 (element e in the
// low half of word e/2 for even e).  Each conversion is gfx950's
// v_cvt_pk_bf16_f32 (two floats to their nearest bfloat16 values, ties to
// even, in the default rounding mode); widening a bfloat16 back to float is
// exact, and so is each residual: x minus its nearest 8-bit value needs at
// most 16 significant bits, and that residual minus its own nearest 8-bit
// value at most 8.
__device__ __forceinline__ void split8(const float v[8], u32x4 out[3]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 x = {v[2 * w], v[2 * w + 1]};
    const bf16x2 h0 = __builtin_convertvector(x, bf16x2);
    const f32x2 r1 = x - __builtin_convertvector(h0, f32x2);
    const bf16x2 h1 = __builtin_convertvector(r1, bf16x2);
    const f32x2 r2 = r1 - __builtin_convertvector(h1, f32x2);
    const bf16x2 h2 = __builtin_convertvector(r2, bf16x2);
    out[0][w] = __builtin_bit_cast(unsigned, h0);
    out[1][w] = __builtin_bit_cast(unsigned, h1);
    out[2][w] = __builtin_bit_cast(unsigned, h2);
  }
}

// ------------------------------------------------------------------ split
// One launch splits both operands: work-groups [0, blocks_a) take A, the
// rest take B.  Each operand is split one of two ways, by where its k runs:
//
// k along the stored columns (A as given, B transposed; rows x K, leading
// dimension ld): one thread per 8 consecutive k of one row, k >= K read as 0.
// A work-group covers 256 / CW rows by CW such chunks (CW = 2^lcw, the
// chunks per row rounded up to a power of two, at most 64), so a thread's
// row and chunk come from shifts of its index.  VEC: 16-byte aligned base
// and ld % 4 == 0, so the 8 values come in two 16-byte loads where they lie
// inside the row.
//
// k along the stored rows (B as given, A transposed; K x cols), written
// transposed as [cols][Kp]: a 64 (k) x 64 (column) tile goes through LDS
// (read as 16 float4 per k row where VEC: 16-byte aligned, ld % 4 == 0,
// cols % 4 == 0); then lane l of each group of 8 takes k-chunk l % 8 of one
// column, so 8 lanes write 128 contiguous bytes of a plane row.
constexpr int kSplitT = 64;

struct SplitOperand {
  const float *X;
  long ld;
  int rows;     // rows of the planes: M for A, N for B
  bool kcols;   // k runs along the stored columns
  u32x4 *w;     // plane 0 (16-byte chunks); planes are rows * Kp / 8 chunks apart
  long blocks;  // work-groups of this operand
  int tiles_c;  // k-along-rows split: 64-column tiles
  int lcw;      // k-along-columns split: log2 of the chunks per work-group row
  int groups_c; // k-along-columns split: work-groups across one row's chunks
};

struct SplitArgs {
  SplitOperand a, b;
  int K, Kp;
};

template <bool VEC>
__device__ __forceinline__ void split_kcols_part(const SplitOperand &o, int K, int Kp, long blk) {
  const int cpr = Kp / 8;
  const long plane = (long)o.rows * cpr;
  const int by = (int)(blk / o.groups_c), bx = (int)(blk % o.groups_c);  // uniform
  const int tid = threadIdx.x;
  const int row = (by << (8 - o.lcw)) + (tid >> o.lcw);
  const int c = (bx << o.lcw) + (tid & ((1 << o.lcw) - 1));
  if (row >= o.rows || c >= cpr) return;
  const long q = (long)row * cpr + c;
  const int k0 = c * 8;
  const float *x = o.X + (long)row * o.ld + k0;
  float v[8];
  if (VEC && k0 + 8 <= K) {
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(x);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(x + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = lo[e];
      v[4 + e] = hi[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = k0 + e < K ? x[e] : 0.f;
  }
  u32x4 out[3];
  split8(v, out);
#pragma unroll
  for (int pl = 0; pl < 3; ++pl) o.w[pl * plane + q] = out[pl];
}

template <bool VEC>
__device__ __forceinline__ void split_krows_part(const SplitOperand &o, int K, int Kp, long blk,
                                                 float (*tile)[kSplitT + 1]) {
  const int tid = threadIdx.x;
  const int cols = o.rows;
  const int tn = (int)(blk % o.tiles_c), tk = (int)(blk / o.tiles_c);
  const int n0 = tn * kSplitT, k0 = tk * kSplitT;
  if constexpr (VEC) {
    // 64 rows x 16 float4: 4 per thread.
#pragma unroll
    for (int i = 0; i < kSplitT * kSplitT / 4 / 256; ++i) {
      const int f = tid + i * 256;
      const int r = f / (kSplitT / 4), c4 = (f % (kSplitT / 4)) * 4;
      const int k = k0 + r, n = n0 + c4;
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      if (k < K && n < cols) t = *reinterpret_cast<const f32x4 *>(o.X + (long)k * o.ld + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[r][c4 + e] = t[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSplitT * kSplitT / 256; ++i) {
      const int r = tid / kSplitT + i * (256 / kSplitT), c = tid % kSplitT;
      const int k = k0 + r, n = n0 + c;
      tile[r][c] = (k < K && n < cols) ? o.X[(long)k * o.ld + n] : 0.f;
    }
  }
  __syncthreads();
  const int cpr = Kp / 8;
  const long plane = (long)cols * cpr;
#pragma unroll
  for (int i = 0; i < kSplitT * (kSplitT / 8) / 256; ++i) {
    const int task = tid + i * 256;
    const int kc = task % 8, c = task / 8;
    const int n = n0 + c, kchunk = k0 / 8 + kc;
    if (n >= cols || kchunk >= cpr) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[kc * 8 + e][c];
    u32x4 out[3];
    split8(v, out);
    const long q = (long)n * cpr + kchunk;
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) o.w[pl * plane + q] = out[pl];
  }
}

template <bool VA, bool VB>
__global__ void __launch_bounds__(256) split_kernel(SplitArgs p) {
  __shared__ float tile[kSplitT][kSplitT + 1];
  const long blk = blockIdx.x;
  // Which operand and which kind are uniform over the work-group.
  if (blk < p.a.blocks) {
    if (p.a.kcols)
      split_kcols_part<VA>(p.a, p.K, p.Kp, blk);
    else
      split_krows_part<VA>(p.a, p.K, p.Kp, blk, tile);
  } else {
    if (p.b.kcols)
      split_kcols_part<VB>(p.b, p.K, p.Kp, blk - p.a.blocks);
    else
      split_krows_part<VB>(p.b, p.K, p.Kp, blk - p.a.blocks, tile);
  }
}

static SplitOperand split_operand(const float *X, long ld, int rows, bool kcols, int Kp,
                                  void *w, bool &vec) {
  SplitOperand o;
  o.X = X;
  o.ld = ld;
  o.rows = rows;
  o.kcols = kcols;
  o.w = reinterpret_cast<u32x4 *>(w);
  o.tiles_c = (rows + kSplitT - 1) / kSplitT;
  const int cpr = Kp / 8;
  o.lcw = 0;
  while ((1 << o.lcw) < cpr && o.lcw < 6) ++o.lcw;
  o.groups_c = (cpr + (1 << o.lcw) - 1) >> o.lcw;
  if (kcols) {
    const int rows_per_group = 256 >> o.lcw;
    o.blocks = (long)((rows + rows_per_group - 1) / rows_per_group) * o.groups_c;
  } else {
    o.blocks = (long)o.tiles_c * ((Kp + kSplitT - 1) / kSplitT);
  }
  vec = (reinterpret_cast<uintptr_t>(X) & 15u) == 0 && ld % 4 == 0 && (kcols || rows % 4 == 0);
  return o;
}

hipError_t launch_split(bool ta, bool tb, const float *A, long lda, const float *B, long ldb,
                        int M, int N, int K, int Kp, void *wa, void *wb, hipStream_t stream) {
  SplitArgs p;
  bool va, vb;
  p.a = split_operand(A, lda, M, !ta, Kp, wa, va);
  p.b = split_operand(B, ldb, N, tb, Kp, wb, vb);
  p.K = K;
  p.Kp = Kp;
  const dim3 grid((unsigned)(p.a.blocks + p.b.blocks)), block(256);
  if (va && vb)
    hipLaunchKernelGGL((split_kernel<true, true>), grid, block, 0, stream, p);
  else if (va)
    hipLaunchKernelGGL((split_kernel<true, false>), grid, block, 0, stream, p);
  else if (vb)
    hipLaunchKernelGGL((split_kernel<false, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((split_kernel<false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- product
// Chunk swizzle of the bfloat16 slice images: row `row` of BK values has
// BK/8 16-byte chunks; chunk c is stored at c ^ swz(row).  With 32-byte rows
// (BK = 16) swz = bit 2 ^ bit 3 of the row, with 64-byte rows (BK = 32) the
// FP32 kernel's 4-chunk swizzle: either way the 128-bit operand reads of 8
// and of 16 consecutive rows fall on disjoint banks.
template <int BK>
__device__ __forceinline__ int bf16_swizzle(int row) {
  static_assert(BK == 16 || BK == 32, "16 or 32 bfloat16 per slice row");
  if constexpr (BK == 16)
    return ((row >> 2) ^ (row >> 3)) & 1;
  else
    return kc_swizzle<16, true>(row);
}

// NS LDS stages: slice t lives in stage t % NS; the loads of slice t + NS
// go out right after the barrier that ends slice t, so each load has NS - 1
// slices of time to arrive.
//
// Software pipeline (MODE):
//   0  per k step: read the three planes' fragments, then the six products;
//   1  the next k step's fragments are read before this step's products are
//      issued (two full fragment sets live);
//   2  plane by plane: plane 1 is read while the plane-0 product runs, plane
//      2 while the two products of order 1 run, and the next k step's plane
//      0 while the three of order 2 run (four plane sets live).
template <int BM, int BN, int BK, int WM, int WN, int MODE, int NS>
__global__ void __launch_bounds__(WM *WN *kWave)
bf16x3_gemm_kernel(Bf16x3Args p, TileMap tmap) {
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR = BK / 8;              // 16-byte chunks per image row
  constexpr int KS = BK / 16;              // matrix-core k steps per slice
  constexpr int NBA = BM * BK * 2 / 1024;  // 1 KiB loads per plane of A
  constexpr int NBB = BN * BK * 2 / 1024;
  static_assert(NBA % NW == 0 && NBB % NW == 0, "loads must split evenly over the waves");
  constexpr int QA = NBA / NW, QB = NBB / NW;  // loads per wave per plane
  constexpr int PA = BM * BK, PB = BN * BK;    // bfloat16 per plane image

  constexpr int LPS = 3 * (QA + QB);           // loads per wave per slice
  static_assert(LPS * (NS - 1) < 64, "outstanding loads must fit vmcnt");

  __shared__ __attribute__((aligned(1024))) unsigned short As0[3 * PA];
  __shared__ __attribute__((aligned(1024))) unsigned short As1[3 * PA];
  __shared__ __attribute__((aligned(1024))) unsigned short As2[NS > 2 ? 3 * PA : 8];
  __shared__ __attribute__((aligned(1024))) unsigned short As3[NS > 3 ? 3 * PA : 8];
  __shared__ __attribute__((aligned(1024))) unsigned short Bs0[3 * PB];
  __shared__ __attribute__((aligned(1024))) unsigned short Bs1[3 * PB];
  __shared__ __attribute__((aligned(1024))) unsigned short Bs2[NS > 2 ? 3 * PB : 8];
  __shared__ __attribute__((aligned(1024))) unsigned short Bs3[NS > 3 ? 3 * PB : 8];
  auto stage_a = [&](auto S) -> unsigned short * {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return As0;
    else if constexpr (st == 1) return As1;
    else if constexpr (st == 2) return As2;
    else return As3;
  };
  auto stage_b = [&](auto S) -> unsigned short * {
    constexpr int st = decltype(S)::value;
    if constexpr (st == 0) return Bs0;
    else if constexpr (st == 1) return Bs1;
    else if constexpr (st == 2) return Bs2;
    else return Bs3;
  };

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane % 32, half = lane / 32;

  int bidx, tm, tn;  // one product: bidx is 0
  tmap.tile(xcd_contiguous_id(blockIdx.x, gridDim.x), bidx, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const long Kp = p.Kp;

  // Lane offsets (bytes from the slice origin of a plane), shared by the
  // three planes; rows past M (N) read as zeros.
  unsigned offA[QA], offB[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int f = (wave + q * NW) * kWave + lane;
    const int row = f / CPR, c = (f % CPR) ^ bf16_swizzle<BK>(row);
    offA[q] = m0 + row < p.M ? (unsigned)((row * Kp + c * 8) * 2) : kOutOfRange;
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int f = (wave + q * NW) * kWave + lane;
    const int row = f / CPR, c = (f % CPR) ^ bf16_swizzle<BK>(row);
    offB[q] = n0 + row < p.N ? (unsigned)((row * Kp + c * 8) * 2) : kOutOfRange;
  }

  const int nk = (int)(Kp / BK);
  auto dma = [&](auto S, int t) {
    unsigned short *as = stage_a(S);
    unsigned short *bs = stage_b(S);
    const long k0 = t < nk ? (long)t * BK : 0;
    const int records = t < nk ? kBufferRecords : 0;
#pragma unroll
    for (int pl = 0; pl < 3; ++pl) {
      const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned short *>(p.a + pl * p.plane_a + (long)m0 * Kp + k0), 0, records,
          kRawBufferWord3);
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned short *>(p.b + pl * p.plane_b + (long)n0 * Kp + k0), 0, records,
          kRawBufferWord3);
#pragma unroll
      for (int q = 0; q < QA; ++q)
        lds_dma<true>(ra, reinterpret_cast<float *>(as + pl * PA + (wave + q * NW) * 512), offA[q]);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        lds_dma<true>(rb, reinterpret_cast<float *>(bs + pl * PB + (wave + q * NW) * 512), offB[q]);
    }
  };

  // Fragments of one plane for k step j: lane reads row (wave row base +
  // i*32 + r32), logical chunk 2j + half.  The row's swizzle depends only on
  // r32 (row mod 16).
  const int sw = bf16_swizzle<BK>(r32);
  struct Plane {
    bf16x8 a[FM];
    bf16x8 b[FN];
  };
  auto read = [&](auto S, int j, int pl, Plane &d) {
    const unsigned short *as = stage_a(S) + pl * PA;
    const unsigned short *bs = stage_b(S) + pl * PB;
    const int ch = ((2 * j + half) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      d.a[i] = *reinterpret_cast<const bf16x8 *>(as + (wm * WTM + i * 32 + r32) * BK + ch);
#pragma unroll
    for (int i = 0; i < FN; ++i)
      d.b[i] = *reinterpret_cast<const bf16x8 *>(bs + (wn * WTN + i * 32 + r32) * BK + ch);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // acc += (a pieces of x) (b pieces of y)
  auto mma = [&](const Plane &x, const Plane &y) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16_bf16(x.a[i], y.b[j], acc[i][j]);
  };

  using S0 = std::integral_constant<int, 0>;
  Plane c0, c1, c2, n0p, n1p, n2p;

  // Slice t is in stage S = t % NS; slice t + 1 is in (or on its way to) SN.
  // The barrier that ends the slice waits until slice t + 1 has landed (the
  // loads of the NS - 2 slices after it may stay in flight).
  auto end_barrier = [&]() { dma_barrier_keep<LPS * (NS - 2)>(); };
  auto slice = [&](auto S, int t) {
    constexpr int s = decltype(S)::value;
    using SN = std::integral_constant<int, (s + 1) % NS>;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bool last = j + 1 == KS;
      if constexpr (MODE == 0) {
        read(S, j, 0, c0);
        read(S, j, 1, c1);
        read(S, j, 2, c2);
        if (last) {
          end_barrier();
          dma(S, t + NS);
        }
        mma(c0, c0);
        mma(c0, c1);
        mma(c1, c0);
        mma(c0, c2);
        mma(c1, c1);
        mma(c2, c0);
      } else if constexpr (MODE == 1) {
        if (!last) {
          read(S, j + 1, 0, n0p);
          read(S, j + 1, 1, n1p);
          read(S, j + 1, 2, n2p);
        } else {
          end_barrier();
          dma(S, t + NS);
          read(SN(), 0, 0, n0p);  // harmless if there is no slice t+1
          read(SN(), 0, 1, n1p);
          read(SN(), 0, 2, n2p);
        }
        mma(c0, c0);
        mma(c0, c1);
        mma(c1, c0);
        mma(c0, c2);
        mma(c1, c1);
        mma(c2, c0);
        c0 = n0p;
        c1 = n1p;
        c2 = n2p;
      } else {
        read(S, j, 1, c1);
        mma(c0, c0);
        read(S, j, 2, c2);
        mma(c0, c1);
        mma(c1, c0);
        if (!last) {
          read(S, j + 1, 0, n0p);
        } else {
          end_barrier();
          dma(S, t + NS);
          read(SN(), 0, 0, n0p);  // harmless if there is no slice t+1
        }
        mma(c0, c2);
        mma(c1, c1);
        mma(c2, c0);
        c0 = n0p;
      }
    }
  };

  dma(S0(), 0);
  dma(std::integral_constant<int, 1>(), 1);
  if constexpr (NS > 2) dma(std::integral_constant<int, 2 % NS>(), 2);
  if constexpr (NS > 3) dma(std::integral_constant<int, 3 % NS>(), 3);
  dma_barrier_keep<LPS * (NS - 1)>();  // slice 0 has landed
  if constexpr (MODE == 1) {
    read(S0(), 0, 0, c0);
    read(S0(), 0, 1, c1);
    read(S0(), 0, 2, c2);
  } else if constexpr (MODE == 2) {
    read(S0(), 0, 0, c0);
  }
  for (int t = 0; t < nk; t += NS) {
    slice(S0(), t);
    if (t + 1 < nk) slice(std::integral_constant<int, 1>(), t + 1);
    if constexpr (NS > 2)
      if (t + 2 < nk) slice(std::integral_constant<int, 2 % NS>(), t + 2);
    if constexpr (NS > 3)
      if (t + 3 < nk) slice(std::integral_constant<int, 3 % NS>(), t + 3);
  }
  // The last slices issued loads past K (zero-filling, no memory traffic);
  // let them retire before the work-group gives up its LDS.
  __builtin_amdgcn_s_waitcnt(0x0f70);

  // Epilogue as in the FP32 kernel: C is read only when beta != 0 (a
  // block's 16 values per lane all loaded before any store); other stores
  // are non-temporal.
  const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN + r32;
  const bool full = (m0 + BM <= p.M) && (n0 + BN <= p.N);
  const bool plain = p.alpha == 1.f && p.beta == 0.f;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + j * 32;
      auto row = [&](int e) { return row0 + i * 32 + acc32_row(lane, e); };
      auto inside = [&](int e) { return full || (row(e) < p.M && col < p.N); };
      auto at = [&](int e) { return p.C + (long)row(e) * p.ldc + col; };
      if (plain) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (inside(e)) __builtin_nontemporal_store(acc[i][j][e], at(e));
      } else if (p.beta == 0.f) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (inside(e)) __builtin_nontemporal_store(p.alpha * acc[i][j][e], at(e));
      } else {
        float c[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) c[e] = inside(e) ? *at(e) : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (inside(e)) *at(e) = fmaf(p.alpha, acc[i][j][e], p.beta * c[e]);
      }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int MODE, int NS>
static hipError_t launch_bf16x3_cfg(const Bf16x3Args &p, hipStream_t stream) {
  if (!dma_offsets_fit(BM, p.Kp / 2, BN, p.Kp / 2)) return hipErrorInvalidValue;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  hipLaunchKernelGGL((bf16x3_gemm_kernel<BM, BN, BK, WM, WN, MODE, NS>),
                     dim3((unsigned)((long)tiles_m * tiles_n)), dim3(WM * WN * kWave), 0, stream,
                     p, make_tile_map(tiles_m, tiles_n, 8));
  return hipGetLastError();
}

// Tile of the six-product kernel: the largest of 256 x 256 and 128 x 128
// that still gives every compute unit a work-group and whose tiles lie at
// least 3/4 inside C; else 64 x 64.
hipError_t launch_bf16x3_gemm(const Bf16x3Args &p, int cus, hipStream_t stream) {
  auto tiles = [&](long t) { return (double)((p.M + t - 1) / t) * ((p.N + t - 1) / t); };
  auto good = [&](long t) {
    return tiles(t) >= cus && 4.0 * p.M * p.N >= 3.0 * tiles(t) * t * t;
  };
  if (good(256)) return launch_bf16x3_cfg<256, 256, 16, 2, 4, 0, 2>(p, stream);
  if (good(128)) return launch_bf16x3_cfg<128, 128, 32, 2, 4, 1, 2>(p, stream);
  return launch_bf16x3_cfg<64, 64, 32, 2, 2, 1, 2>(p, stream);
}

// One-instruction probe of v_mfma_f32_32x32x16_bf16: A is 32 x 16 and B is
// 16 x 32, row-major floats that are exact bfloat16 values (their high
// halves are taken); C is 32 x 32 row-major.
__global__ void __launch_bounds__(kWave) bf16_probe_kernel(const float *A, const float *B,
                                                          float *C) {
  const int l = threadIdx.x;
  bf16x8 a, b;
  unsigned short ha[8], hb[8];
  for (int e = 0; e < 8; ++e) {
    ha[e] = (unsigned short)(__float_as_uint(A[(l % 32) * 16 + 8 * (l / 32) + e]) >> 16);
    hb[e] = (unsigned short)(__float_as_uint(B[(8 * (l / 32) + e) * 32 + l % 32]) >> 16);
  }
  __builtin_memcpy(&a, ha, sizeof a);
  __builtin_memcpy(&b, hb, sizeof b);
  f32x16 acc;
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  acc = mfma32x32x16_bf16(a, b, acc);
  for (int e = 0; e < 16; ++e) C[acc32_row(l, e) * 32 + l % 32] = acc[e];
}

hipError_t launch_bf16_probe(const float *A, const float *B, float *C, hipStream_t stream) {
  hipLaunchKernelGGL(bf16_probe_kernel, dim3(1), dim3(kWave), 0, stream, A, B, C);
  return hipGetLastError();
}

}  // namespace sgemm
