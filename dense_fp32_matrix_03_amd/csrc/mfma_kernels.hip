// mfma_kernels.hip -- single-precision matrix product on the gfx950 matrix
// cores (v_mfma_f32_32x32x2_f32), plus the one-instruction layout probe.
//
// Structure (the pages' recipe, re-derived for CDNA4):
//  * block tiling with a K-sliding window: each work-group owns a BM x BN tile
//    of C and walks K in BK-wide slices (textbook chapter "4. 矩阵乘法性能优化",
//    section 一);
//  * each slice of A (BM x BK) and B (BK x BN) is fetched once with coalesced
//    128-bit loads and staged in LDS (chapter section 三; article
//    "硬件加速原理：CUDA核函数优化矩阵乘法的内存访问模式", section
//    "内存合并访问原理");
//  * two LDS stages: the global loads of slice t+1 are issued before the
//    matrix-core work of slice t and written to the other stage after it, one
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
// lane's A operands for a whole slice are BK/2 consecutive floats of one
// LDS row, read with 128-bit LDS loads.  A's LDS rows are padded by 4 floats
// (row stride BK + 4 = 20 words for BK = 16): eight consecutive rows then
// start 20 banks apart and a 128-bit read by rows r .. r+7 touches 32
// distinct banks.  B stays row-major in LDS; its operand reads are 32-bit,
// consecutive lanes on consecutive banks.
#include "common.hpp"
#include "dispatch.hpp"

namespace sgemm {

template <int BM, int BN, int BK, int WM, int WN, int APAD, bool VA, bool VB>
__global__ void __launch_bounds__(WM *WN *kWave)
mfma_gemm_kernel(GemmArgs p, int tiles_m, int tiles_n, int group_m) {
  constexpr int NT = WM * WN * kWave;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 blocks per wave
  constexpr int KH = BK / 2;                   // matrix-core steps per slice
  constexpr int SA = BK + APAD;                // LDS row stride of the A slice
  constexpr int SB = BN;                       // LDS row stride of the B slice
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(KH % 4 == 0, "BK must be a multiple of 8");
  static_assert(SA % 4 == 0, "A rows must stay 16-byte aligned in LDS");

  using FetchA = SliceFetch<BM, BK, NT, VA>;
  using FetchB = SliceFetch<BK, BN, NT, VB>;

  __shared__ __attribute__((aligned(16))) float As[2][BM * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane % 32, half = lane / 32;

  int tm, tn;
  grouped_tile(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, group_m, tm, tn);
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

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute_slice = [&](int s) {
    const float *as = &As[s][(wm * WTM + r32) * SA + half * KH];
    const float *bs = &Bs[s][(half * KH) * SB + wn * WTN + r32];
#pragma unroll
    for (int kk = 0; kk < KH; kk += 4) {
      f32x4 a[FM];
      float b[FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const f32x4 *>(as + i * 32 * SA + kk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t) b[j][t] = bs[(kk + t) * SB + j * 32];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x2(a[i][t], b[j][t], acc[i][j]);
    }
  };

  const int nk = (p.K + BK - 1) / BK;
  fa.load(p.M, p.K);
  fb.load(p.K, p.N);
  store_slice(0);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const bool more = t + 1 < nk;
    if (more) {
      fa.advance(0, BK);
      fb.advance(BK, 0);
      fa.load(p.M, p.K);
      fb.load(p.K, p.N);
    }
    compute_slice(t & 1);
    if (more) store_slice((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: register j of lane l holds row acc32_row(l, j), column l % 32
  // of its 32x32 block; rows >= M and columns >= N are not stored.
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

// One configuration of the kernel: block tile, wave grid, slice depth.
template <int BM, int BN, int BK, int WM, int WN, int APAD>
static hipError_t launch_cfg(const GemmArgs &p, bool va, bool vb, hipStream_t stream) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const long nwg = (long)tiles_m * tiles_n;
  const dim3 grid((unsigned)nwg), block(WM * WN * kWave);
  const int group_m = 8;
  if (va && vb)
    hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WM, WN, APAD, true, true>), grid, block, 0,
                       stream, p, tiles_m, tiles_n, group_m);
  else if (va)
    hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WM, WN, APAD, true, false>), grid, block, 0,
                       stream, p, tiles_m, tiles_n, group_m);
  else if (vb)
    hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WM, WN, APAD, false, true>), grid, block, 0,
                       stream, p, tiles_m, tiles_n, group_m);
  else
    hipLaunchKernelGGL((mfma_gemm_kernel<BM, BN, BK, WM, WN, APAD, false, false>), grid, block, 0,
                       stream, p, tiles_m, tiles_n, group_m);
  return hipGetLastError();
}

hipError_t launch_mfma(MfmaTile tile, const GemmArgs &p, bool va, bool vb, hipStream_t stream) {
  switch (tile) {
    case MfmaTile::T256: return launch_cfg<256, 256, 16, 2, 2, 4>(p, va, vb, stream);
    case MfmaTile::T128: return launch_cfg<128, 128, 16, 2, 2, 4>(p, va, vb, stream);
    case MfmaTile::T64: return launch_cfg<64, 64, 16, 2, 2, 4>(p, va, vb, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Layout probe: one wave, one matrix-core instruction, packed row-major
// operands; the accumulator is written back through the lane map above.
__global__ void __launch_bounds__(kWave) mfma_probe_kernel(int which, const float *A,
                                                            const float *B, float *C) {
  const int l = threadIdx.x;
  if (which == 0) {
    // A is 32 x 2, B is 2 x 32.
    const float a = A[(l % 32) * 2 + l / 32];
    const float b = B[(l / 32) * 32 + l % 32];
    f32x16 acc;
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    acc = mfma32x32x2(a, b, acc);
    for (int e = 0; e < 16; ++e) C[acc32_row(l, e) * 32 + l % 32] = acc[e];
  } else {
    // A is 16 x 4, B is 4 x 16.
    const float a = A[(l % 16) * 4 + l / 16];
    const float b = B[(l / 16) * 16 + l % 16];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma16x16x4(a, b, acc);
    for (int e = 0; e < 4; ++e) C[(4 * (l / 16) + e) * 16 + l % 16] = acc[e];
  }
}

hipError_t launch_mfma_probe(int which, const float *A, const float *B, float *C,
                             hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(kWave), 0, stream, which, A, B, C);
  return hipGetLastError();
}

}  // namespace sgemm
