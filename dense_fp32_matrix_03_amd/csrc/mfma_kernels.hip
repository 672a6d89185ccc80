// mfma_kernels.hip -- the configurations of the matrix-core kernels that the
// library dispatches to, and the one-instruction layout probe.
#include "common.hpp"
#include "dispatch.hpp"
#include "mfma_dma.hpp"
#include "mfma_gemm.hpp"

namespace sgemm {

// Tile configurations (block tile, K slice, wave grid), from a sweep over
// square problems of 1024 .. 8192 on MI355X:
//   T256  256 x 256 x 32, 2 x 4 waves of 128 x 64  (two waves per SIMD)
//   T128  128 x 128 x 32, 4 x 2 waves of  32 x 64  (two waves per SIMD;
//         the register-staged kernel keeps 2 x 2 waves of 64 x 64)
//   T64    64 x  64 x 32, 2 x 2 waves of  32 x 32
//   T32    32 x  32 x 32, 4 waves on the same 32 x 32 block, each taking
//         one of the four k groups of every slice (KSPLIT = 4); for
//         products with at most 3/4 as many 64 x 64 tiles as CUs it spreads
//         the work over four times as many work-groups, each on four SIMDs
//         (512^3: 11.7 -> 7.3 us; 640 x 640 x 2048: 35.4 -> 26.5 us).
// At 2048^3 (one 128 x 128 tile per CU) eight waves instead of four took the
// buffer-to-LDS kernel from 140.7 to 144.9 TFLOP/s; at 4096^3 both give 150.5.
// WIDE_ONLY: only the 16-byte-load forms are instantiated (the caller
// guarantees va && vb).  DWM x DWN: wave grid of the buffer-to-LDS kernel.
template <int BM, int BN, int BK, int WM, int WN, bool WIDE_ONLY = false, int DWM = WM,
          int DWN = WN>
static hipError_t launch_tile(MfmaPath path, const GemmArgs &p, bool va, bool vb,
                              hipStream_t stream) {
  constexpr int kStoreGroup = 1;  // staged kernel: write the next slice after group 1 of 4
  const bool dma = dma_offsets_fit(BM, p.lda, BK, p.ldb);
  switch (path) {
    case MfmaPath::Auto:
      if (dma) return launch_dma_cfg<BM, BN, BK, DWM, DWN, true, 1, WIDE_ONLY>(p, va, vb, stream);
      return launch_staged_cfg<BM, BN, BK, WM, WN, 4, kStoreGroup>(p, va, vb, stream);
    case MfmaPath::Unpadded:
      if (dma) return launch_dma_cfg<BM, BN, BK, DWM, DWN, false, 1, WIDE_ONLY>(p, va, vb, stream);
      return launch_staged_cfg<BM, BN, BK, WM, WN, 0, kStoreGroup>(p, va, vb, stream);
    case MfmaPath::Staged:
      return launch_staged_cfg<BM, BN, BK, WM, WN, 4, kStoreGroup>(p, va, vb, stream);
  }
  return hipErrorInvalidValue;
}

// The largest tile that still gives every compute unit a work-group and
// whose tiles are at least 3/4 inside C (a 256 x 256 tile over a 64 x 64
// product would compute 16 times the useful work); else 64 x 64, unless its
// tiles would leave more than a quarter of the compute units idle: then the
// k-split 32 x 32 tile.  (Four 32 x 32 work-groups per 64 x 64 tile; at 3/4
// of the CUs or fewer they fit in three rounds where 64 x 64 needs one full
// round each, and the measured crossover lies between 192 and 208 tiles on
// 256 CUs.)
MfmaTile choose_mfma_tile(long M, long N, int cus, long batch) {
  auto tiles = [&](long t) { return (double)((M + t - 1) / t) * ((N + t - 1) / t) * batch; };
  auto good = [&](long t) {
    return tiles(t) >= cus && 4.0 * M * N * batch >= 3.0 * tiles(t) * t * t;
  };
  if (good(256)) return MfmaTile::T256;
  if (good(128)) return MfmaTile::T128;
  return 4.0 * tiles(64) <= 3.0 * cus ? MfmaTile::T32 : MfmaTile::T64;
}

hipError_t launch_mfma(MfmaTile tile, MfmaPath path, const GemmArgs &p, bool va, bool vb,
                       hipStream_t stream) {
  switch (tile) {
    case MfmaTile::T256:
      // The 256 x 256 tile keeps 128 accumulators per lane; its 4-byte-load
      // forms would spill, so operands that need them take the 128 x 128 tile.
      if (!(va && vb)) return launch_tile<128, 128, 32, 2, 2, false, 4, 2>(path, p, va, vb, stream);
      return launch_tile<256, 256, 32, 2, 4, true>(path, p, va, vb, stream);
    case MfmaTile::T128:
      return launch_tile<128, 128, 32, 2, 2, false, 4, 2>(path, p, va, vb, stream);
    case MfmaTile::T64: return launch_tile<64, 64, 32, 2, 2>(path, p, va, vb, stream);
    case MfmaTile::T32:
      // The register-staged kernel has no k split: it takes the 64 x 64 tile.
      if (path == MfmaPath::Staged || !dma_offsets_fit(32, p.lda, 32, p.ldb))
        return launch_tile<64, 64, 32, 2, 2>(path, p, va, vb, stream);
      if (path == MfmaPath::Unpadded)
        return launch_dma_cfg<32, 32, 32, 1, 1, false, 1, false, 4>(p, va, vb, stream);
      return launch_dma_cfg<32, 32, 32, 1, 1, true, 1, false, 4>(p, va, vb, stream);
  }
  return hipErrorInvalidValue;
}

template <int BM, int BN, int BK, int WM, int WN, int KSPLIT = 1>
static hipError_t launch_general_tile(const GemmArgs &p, bool ta, bool tb, bool va, bool vb,
                                      hipStream_t stream) {
  if (!dma_offsets_fit(ta ? BK : BM, p.lda, tb ? BN : BK, p.ldb)) return hipErrorInvalidValue;
  return launch_dma_general<BM, BN, BK, WM, WN, KSPLIT>(p, ta, tb, va, vb, stream);
}

hipError_t launch_mfma_general(MfmaTile tile, const GemmArgs &p, bool ta, bool tb, bool va,
                               bool vb, hipStream_t stream) {
  // The 256 x 256 tile is instantiated for the plain layout with 16-byte
  // loads only (other forms would spill); the rest use 128 x 128.
  if (tile == MfmaTile::T256 && !ta && !tb && va && vb) {
    if (!dma_offsets_fit(256, p.lda, 32, p.ldb)) return hipErrorInvalidValue;
    return launch_dma_cfg<256, 256, 32, 2, 4, true, 1, true>(p, va, vb, stream);
  }
  if (tile == MfmaTile::T64) return launch_general_tile<64, 64, 32, 2, 2>(p, ta, tb, va, vb, stream);
  if (tile == MfmaTile::T32)
    return launch_general_tile<32, 32, 32, 1, 1, 4>(p, ta, tb, va, vb, stream);
  return launch_general_tile<128, 128, 32, 4, 2>(p, ta, tb, va, vb, stream);
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
