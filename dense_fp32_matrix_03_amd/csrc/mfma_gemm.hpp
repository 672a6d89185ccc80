// mfma_gemm.hpp -- register-staged matrix-core product (v_mfma_f32_32x32x2_f32).
//
// sgemm_run uses the buffer-to-LDS kernel of mfma_dma.hpp for every operand
// whose K slice fits a buffer descriptor (aligned or not); this kernel takes
// the rest -- a leading dimension so large that one slice spans 2 GiB -- and
// is the register-staged ablation variant.  Any 4-byte alignment, any
// leading dimension.
//
// Structure (the pages' recipe, re-derived for CDNA4):
//  * block tiling with a K-sliding window: each work-group owns a BM x BN tile
//    of C and walks K in BK-wide slices (textbook chapter "4. 矩阵乘法性能优化",
//    section 一);
//  * each slice of A (BM x BK) and B (BK x BN) is fetched once with coalesced
//    loads (128-bit where alignment allows) and staged in LDS (chapter
//    section 三; article "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式",
//    section "内存合并访问原理");
//  * two LDS stages: the global loads of slice t+1 go out at the start of
//    slice t and are written to the other stage part-way through it, one
//    barrier per slice (chapter section 四, double buffering);
//  * each wave owns a (BM/WM) x (BN/WN) register tile of 32 x 32 accumulator
//    blocks -- the matrix-core analogue of the chapter's 8 x 8 per-thread
//    register tile (section 二);
//  * out-of-range rows, columns and k are zero-filled on load and never
//    stored (chapter section 三).
//
// Operand order inside a slice.  A 32x32x2 instruction consumes two k values:
// lanes 0-31 supply the first, lanes 32-63 the second.  Any pairing of k
// values is valid as long as A and B use the same one, so in step t lanes
// 0-31 take slice column t and lanes 32-63 take column BK/2 + t.  Then each
// lane's A operands for four steps are four consecutive floats of one LDS
// row, one 128-bit LDS read.  A's LDS rows are padded by APAD floats: with
// BK = 32 and APAD = 4 the row stride is 36 words, so the 128-bit reads of 8
// (or 16) consecutive rows start on disjoint bank groups.  B stays row-major
// in LDS; its operand reads are 32-bit, consecutive lanes on consecutive
// banks.
//
// Software pipeline.  The slice loop is split into G = BK/8 groups of four
// matrix-core steps, and three things overlap:
//  * operands of group g+1 are read from LDS while group g's instructions
//    run, so the matrix pipe does not wait for an LDS read;
//  * across a slice boundary the next slice's first operands are read right
//    after the barrier while the current slice's last group is still being
//    issued from registers, which hides the LDS latency behind the barrier;
//  * the global loads of slice t+1 are written to the other LDS stage after
//    group STORE_G of slice t, early enough that the writes have drained when
//    the barrier is reached.
#pragma once

#include "common.hpp"

namespace sgemm {

template <int BM, int BN, int BK, int WM, int WN, int APAD, int STORE_G, bool VA, bool VB>
__global__ void __launch_bounds__(WM *WN *kWave)
mfma_gemm_staged_kernel(GemmArgs p, TileMap tmap) {
  constexpr int NT = WM * WN * kWave;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KH = BK / 2;
  constexpr int G = KH / 4;
  constexpr int SA = BK + APAD;
  constexpr int SB = BN;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(KH % 4 == 0, "BK must be a multiple of 8");
  static_assert(SA % 4 == 0 && SB % 4 == 0, "LDS rows must stay 16-byte aligned");
  // The next slice must be in LDS before the barrier that ends this slice,
  // which is issued at the start of the last group.
  static_assert(G >= 2 && STORE_G >= 0 && STORE_G <= G - 2, "store point");

  using FetchA = SliceFetch<BM, BK, NT, VA>;
  using FetchB = SliceFetch<BK, BN, NT, VB>;

  __shared__ __attribute__((aligned(16))) float As[2][BM * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane % 32, half = lane / 32;

  int bidx, tm, tn;  // one product: bidx is 0
  tmap.tile(xcd_contiguous_id(blockIdx.x, gridDim.x), bidx, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  FetchA fa;
  FetchB fb;
  fa.init(p.A, p.lda, m0, 0, tid);
  fb.init(p.B, p.ldb, 0, n0, tid);

  auto store_slice = [&](int s) {
#pragma unroll
    for (int i = 0; i < FetchA::CH; ++i)
      *reinterpret_cast<f32x4 *>(&As[s][FetchA::wrow(tid, i) * SA + FetchA::wcol(tid)]) = fa.v[i];
#pragma unroll
    for (int i = 0; i < FetchB::CH; ++i)
      *reinterpret_cast<f32x4 *>(&Bs[s][FetchB::wrow(tid, i) * SB + FetchB::wcol(tid)]) = fb.v[i];
  };

  // Operands of one group: 4 steps x (FM A values + FN B values) per lane.
  struct Ops {
    f32x4 a[FM];
    f32x4 b[FN];
  };
  const int a_off = (wm * WTM + r32) * SA + half * KH;
  const int b_off = (half * KH) * SB + wn * WTN + r32;
  auto read_ops = [&](int s, int g, Ops &o) {
    const float *as = &As[s][a_off + g * 4];
    const float *bs = &Bs[s][b_off + g * 4 * SB];
#pragma unroll
    for (int i = 0; i < FM; ++i) o.a[i] = *reinterpret_cast<const f32x4 *>(as + i * 32 * SA);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) o.b[j][t] = bs[t * SB + j * 32];
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto mma = [&](const Ops &o) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x2(o.a[i][t], o.b[j][t], acc[i][j]);
  };

  const int nk = (p.K + BK - 1) / BK;
  fa.load(p.M, p.K);
  fb.load(p.K, p.N);
  store_slice(0);
  __syncthreads();
  Ops cur, nxt;
  read_ops(0, 0, cur);
  for (int t = 0; t < nk; ++t) {
    const int s = t & 1;
    const bool more = t + 1 < nk;
    if (more) {
      fa.advance(0, BK);
      fb.advance(BK, 0);
      fa.load(p.M, p.K);
      fb.load(p.K, p.N);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g + 1 < G) {
        read_ops(s, g + 1, nxt);
      } else {
        __syncthreads();
        if (more) read_ops(s ^ 1, 0, nxt);
      }
      mma(cur);
      if (g == STORE_G && more) store_slice(s ^ 1);
      cur = nxt;
    }
  }

  const int row0 = m0 + wm * WTM, col0 = n0 + wn * WTN + r32;
  const bool full = (m0 + BM <= p.M) && (n0 + BN <= p.N);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = row0 + i * 32 + acc32_row(lane, e);
        const int col = col0 + j * 32;
        if (full || (row < p.M && col < p.N)) p.C[(long)row * p.ldc + col] = acc[i][j][e];
      }
}

template <int BM, int BN, int BK, int WM, int WN, int APAD, int STORE_G>
inline hipError_t launch_staged_cfg(const GemmArgs &p, bool va, bool vb, hipStream_t stream,
                                  int group_m = 8) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const long nwg = (long)tiles_m * tiles_n;
  const dim3 grid((unsigned)nwg), block(WM * WN * kWave);
  const TileMap tmap = make_tile_map(tiles_m, tiles_n, group_m);
#define SGEMM_STAGED_LAUNCH(VA_, VB_)                                                             \
  hipLaunchKernelGGL(                                                                           \
      (mfma_gemm_staged_kernel<BM, BN, BK, WM, WN, APAD, STORE_G, VA_, VB_>), grid, block, \
      0, stream, p, tmap)
  if (va && vb)
    SGEMM_STAGED_LAUNCH(true, true);
  else if (va)
    SGEMM_STAGED_LAUNCH(true, false);
  else if (vb)
    SGEMM_STAGED_LAUNCH(false, true);
  else
    SGEMM_STAGED_LAUNCH(false, false);
#undef SGEMM_STAGED_LAUNCH
  return hipGetLastError();
}

}  // namespace sgemm
