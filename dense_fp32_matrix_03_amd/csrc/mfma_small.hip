// mfma_small.hip -- products too small to occupy the chip with 32 x 32 tiles.
//
// One work-group of four waves per 16 x 16 tile of C, on the 16x16x4 FP32
// matrix instruction, so that a 256 x 256 product spreads over 256 compute
// units instead of 64.  K is split over the four waves (a k set each), and
// every wave loads all of its operands straight from global memory into
// registers before its first matrix instruction: one memory round trip, no
// LDS staging and no barrier until the four partial sums are added.  The
// LDS-staged kernel (mfma_dma.hpp) spends a workgroup barrier and an LDS
// round trip per K slice; on a product this small those, not the
// arithmetic, set the time.  Each wave reads its own operands, so L2
// traffic grows with the tile count times K, and the tile rule
// (mfma_kernels.hip) keeps this kernel to products whose tiles read little.
//
// k order.  K is walked in chunks of 64 NG values; in a chunk, group g (16
// consecutive k) goes to wave g % 4, and within a group lane quarter h
// supplies k = 16 g + 4 h + t to instruction t (t = 0..3).  A lane's four
// values of op(A) (or op(B)) per group are therefore 4 consecutive k: one
// 16-byte load where the operand's k runs along its stored rows.  The order
// depends on neither the operand layout nor NG (groups past K add exact
// zeros), so stored transposes give the plain layout's bits.  Wave 0 adds the
// other waves' sums in the order 1, 2, 3.
//
// Definition of the product: article "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问
// 模式", section "矩阵乘法的计算特性"; out-of-range elements are zero (textbook
// chapter "4. 矩阵乘法性能优化", section 三).
#include "common.hpp"
#include "dispatch.hpp"

namespace sgemm {

namespace {

constexpr int kSmallTile = 16;
constexpr int kSmallWaves = 4;

// TA / TB: A / B stored transposed.  WA: op(A) takes 16-byte loads (A as
// given, aligned); WB: op(B) takes 16-byte loads (B stored transposed,
// aligned).  Where k runs across an operand's stored rows its four values
// are four 4-byte loads.
template <int NG, bool TA, bool TB, bool WA, bool WB, bool PHASES>
__global__ void __launch_bounds__(kSmallWaves *kWave)
mfma_small_kernel(GemmArgs p, TileMap tmap) {
  auto phase = [&](int i) {
    if constexpr (PHASES) {
      if (threadIdx.x == 0) p.phases[(long)blockIdx.x * 8 + i] = __builtin_amdgcn_s_memrealtime();
    }
  };
  phase(0);
  if constexpr (PHASES) {
    if (threadIdx.x == 0) {
      p.phases[(long)blockIdx.x * 8 + 5] = __builtin_amdgcn_s_memtime();
      p.phases[(long)blockIdx.x * 8 + 7] = (unsigned long long)kSmallTile |
                                           (unsigned long long)kSmallTile << 16 |
                                           (unsigned long long)(64 * NG) << 32 |
                                           (unsigned long long)kSmallWaves << 48;
    }
  }
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane % 16, h = lane / 16;

  // Launch position -> (product of the batch, tile), tiles row by row inside
  // the share of consecutive ids that one XCD receives.
  int bidx, tm, tn;
  tmap.tile(xcd_contiguous_id(blockIdx.x, gridDim.x), bidx, tm, tn);
  const float *Ab = p.A + (long)bidx * p.strideA;
  const float *Bb = p.B + (long)bidx * p.strideB;
  float *Cb = p.C + (long)bidx * p.strideC;
  const int i = tm * kSmallTile + r16;  // row of op(A) this lane loads
  const int j = tn * kSmallTile + r16;  // column of op(B) this lane loads
  const bool row_ok = i < p.M, col_ok = j < p.N;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (long kc = 0; kc < p.K; kc += 64 * NG) {
    f32x4 a[NG], b[NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
      const long k0 = kc + 16 * (w + kSmallWaves * n) + 4 * h;
      if constexpr (WA) {
        // K % 4 == 0 here, so k0 < K covers all four values.
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (row_ok && k0 < p.K) v = *reinterpret_cast<const f32x4 *>(Ab + (long)i * p.lda + k0);
        a[n] = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long k = k0 + q;
          const long off = TA ? k * p.lda + i : (long)i * p.lda + k;
          a[n][q] = row_ok && k < p.K ? Ab[off] : 0.f;
        }
      }
      if constexpr (WB) {
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (col_ok && k0 < p.K) v = *reinterpret_cast<const f32x4 *>(Bb + (long)j * p.ldb + k0);
        b[n] = v;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const long k = k0 + q;
          const long off = TB ? (long)j * p.ldb + k : k * p.ldb + j;
          b[n][q] = col_ok && k < p.K ? Bb[off] : 0.f;
        }
      }
    }
    if constexpr (PHASES) {
      if (kc == 0) {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the first chunk has landed
        phase(1);
      }
    }
#pragma unroll
    for (int n = 0; n < NG; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma16x16x4(a[n][q], b[n][q], acc);
  }
  phase(2);

  // Waves 1..3 leave their sums in LDS; wave 0 adds them in order and stores.
  __shared__ float red[(kSmallWaves - 1) * 4 * kWave];
  if (w > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((w - 1) * 4 + r) * kWave + lane] = acc[r];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int s = 0; s < kSmallWaves - 1; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += red[(s * 4 + r) * kWave + lane];
  phase(3);

  // Register r of lane l holds C(4 (l / 16) + r, l % 16) of the tile.  C is
  // read only when beta != 0; plain stores are non-temporal (C is not read
  // again by this kernel).
  const bool plain = p.alpha == 1.f && p.beta == 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = tm * kSmallTile + 4 * h + r;
    if (row < p.M && col_ok) {
      float *at = Cb + (long)row * p.ldc + j;
      if (plain)
        __builtin_nontemporal_store(acc[r], at);
      else if (p.beta == 0.f)
        __builtin_nontemporal_store(p.alpha * acc[r], at);
      else
        *at = fmaf(p.alpha, acc[r], p.beta * *at);
    }
  }
  if constexpr (PHASES) {
    __builtin_amdgcn_s_waitcnt(0);
    phase(4);
    if (threadIdx.x == 0) p.phases[(long)blockIdx.x * 8 + 6] = __builtin_amdgcn_s_memtime();
  }
}

template <int NG, bool TA, bool TB, bool PHASES>
void launch_ng(const GemmArgs &p, bool wa, bool wb, hipStream_t stream) {
  const int tiles_m = (p.M + kSmallTile - 1) / kSmallTile;
  const int tiles_n = (p.N + kSmallTile - 1) / kSmallTile;
  const dim3 grid((unsigned)((long)tiles_m * tiles_n * p.batch)), block(kSmallWaves * kWave);
  const TileMap tmap = make_tile_map(tiles_m, tiles_n, 1);  // groups of one row: row by row
#define SGEMM_SMALL_LAUNCH(WA_, WB_)                                                        \
  hipLaunchKernelGGL((mfma_small_kernel<NG, TA, TB, WA_, WB_, PHASES>), grid, block, 0, stream, \
                     p, tmap)
  if constexpr (!TA && TB) {
    if (wa && wb) SGEMM_SMALL_LAUNCH(true, true);
    else if (wa) SGEMM_SMALL_LAUNCH(true, false);
    else if (wb) SGEMM_SMALL_LAUNCH(false, true);
    else SGEMM_SMALL_LAUNCH(false, false);
  } else if constexpr (!TA) {
    if (wa) SGEMM_SMALL_LAUNCH(true, false);
    else SGEMM_SMALL_LAUNCH(false, false);
  } else if constexpr (TB) {
    if (wb) SGEMM_SMALL_LAUNCH(false, true);
    else SGEMM_SMALL_LAUNCH(false, false);
  } else {
    SGEMM_SMALL_LAUNCH(false, false);
  }
#undef SGEMM_SMALL_LAUNCH
}

// NG: the smallest of 1, 2, 4, 8, 16 groups per wave that covers K in one
// chunk (K <= 1024); longer K runs in chunks of 1024.
template <bool TA, bool TB, bool PHASES>
void launch_layout(const GemmArgs &p, bool wa, bool wb, hipStream_t s) {
  if (p.K <= 64) launch_ng<1, TA, TB, PHASES>(p, wa, wb, s);
  else if (p.K <= 128) launch_ng<2, TA, TB, PHASES>(p, wa, wb, s);
  else if (p.K <= 256) launch_ng<4, TA, TB, PHASES>(p, wa, wb, s);
  else if (p.K <= 512) launch_ng<8, TA, TB, PHASES>(p, wa, wb, s);
  else launch_ng<16, TA, TB, PHASES>(p, wa, wb, s);
}

}  // namespace

hipError_t launch_small(const GemmArgs &p, bool ta, bool tb, bool va, bool vb,
                        hipStream_t stream) {
  // 16-byte loads serve an operand whose k runs along its stored rows.
  const bool wa = !ta && va, wb = tb && vb;
  if (!ta && !tb) launch_layout<false, false, false>(p, wa, wb, stream);
  else if (!ta) launch_layout<false, true, false>(p, wa, wb, stream);
  else if (!tb) launch_layout<true, false, false>(p, wa, wb, stream);
  else launch_layout<true, true, false>(p, wa, wb, stream);
  return hipGetLastError();
}

hipError_t launch_small_phases(const GemmArgs &p, bool va, hipStream_t stream) {
  launch_layout<false, false, true>(p, va, false, stream);
  return hipGetLastError();
}

long small_workgroups(long M, long N, long batch) {
  return ((M + kSmallTile - 1) / kSmallTile) * ((N + kSmallTile - 1) / kSmallTile) * batch;
}

}  // namespace sgemm
