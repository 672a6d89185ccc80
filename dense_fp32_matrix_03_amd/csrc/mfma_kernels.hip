// mfma_kernels.hip -- the choice of matrix-core configuration for a call,
// the dispatch to the small-product kernel (mfma_small.hip), the per-layout
// launchers of the buffer-to-LDS kernel (mfma_configs.hpp, mfma_layout_*.hip)
// and the register-staged fallback, and the one-instruction layout probe.
#include <math.h>

#include "common.hpp"
#include "dispatch.hpp"
#include "mfma_configs.hpp"

namespace sgemm {

namespace {

struct TileShape {
  MfmaTile tile;
  long bm, bn, threads;
};

// Largest first: the tie-break prefers the larger tile (fewer operand bytes
// per flop, more L2 reuse).
constexpr TileShape kTileShapes[] = {{MfmaTile::T256, 256, 256, 512},
                                     {MfmaTile::T128, 128, 128, 512},
                                     {MfmaTile::T64x96, 64, 96, 768},
                                     {MfmaTile::T64, 64, 64, 512},
                                     {MfmaTile::T32x64, 32, 64, 256},
                                     {MfmaTile::T32, 32, 32, 256},
                                     {MfmaTile::T16, 16, 16, 256}};

// A launch's work-items (work-groups x threads) must fit 32 bits.
constexpr double kMaxWorkItems = 4294967295.0;

long tile_count(long M, long N, long bm, long bn, long batch) {
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * batch;
}

// The share of the matrix-core time that a launch of this tile spends on
// entries of C: every compute unit works through ceil(tiles / cus) tiles of
// bm x bn, of which only M x N per product are wanted.  It is the product of
// the round fill (tiles over rounds x CUs) and the area fill (M N over tiles
// x bm bn); the rest is idle CUs in the last round and padding outside C.
double tile_efficiency(const TileShape &t, long M, long N, int cus, long batch) {
  const double tiles = (double)tile_count(M, N, t.bm, t.bn, batch);
  if (tiles * t.threads > kMaxWorkItems) return 0.0;  // not launchable as one grid
  const double rounds = ceil(tiles / cus);
  return (double)M * N * batch / (rounds * cus * (double)t.bm * (double)t.bn);
}

// DMA configuration of a tile choice; wide: both operands take 16-byte loads
// in the plain layout (the 256 x 256 tile exists only for that form).
DmaCfg dma_cfg(TileChoice t, bool wide_plain) {
  switch (t.tile) {
    case MfmaTile::T256: return wide_plain ? DmaCfg::C256 : DmaCfg::C128;
    case MfmaTile::T128: return DmaCfg::C128;
    case MfmaTile::T64x96: return DmaCfg::C64x96;
    case MfmaTile::T64:
      return !t.ksplit ? DmaCfg::C64 : (t.long_k ? DmaCfg::C64K2L : DmaCfg::C64K2);
    case MfmaTile::T32x64: return t.long_k ? DmaCfg::C32x64L : DmaCfg::C32x64;
    case MfmaTile::T16:  // a variant that runs the buffer-to-LDS kernel instead
    case MfmaTile::T32: return t.long_k ? DmaCfg::C32L : DmaCfg::C32;
  }
  return DmaCfg::C128;
}

// Operand bytes per compute unit that the 16 x 16 tiles read: a 16-row
// strip of op(A) and a 16-column strip of op(B) per tile, each wave loading
// its own share.
double small_bytes_per_cu(long M, long N, long K, int cus, long batch) {
  return (double)tile_count(M, N, 16, 16, batch) * (double)K * (2.0 * 16 * 4) / cus;
}

}  // namespace

bool small_product(long M, long N, long K, int cus, long batch) {
  constexpr long kMaxK = 1024;
  constexpr double kMaxTilesPerCu = 8.0;
  constexpr double kMaxBytesPerCu = 128.0 * 1024;
  return K <= kMaxK && (double)tile_count(M, N, 16, 16, batch) <= kMaxTilesPerCu * cus &&
         small_bytes_per_cu(M, N, K, cus, batch) <= kMaxBytesPerCu;
}

TileChoice with_slice_rule(MfmaTile tile, long M, long N, long K, int cus, long batch) {
  TileChoice c{tile, false, false};
  // The 16 x 16 tile, where a variant runs it on the buffer-to-LDS kernel,
  // takes the 32 x 32 tile's form.
  const MfmaTile form = tile == MfmaTile::T16 ? MfmaTile::T32 : tile;
  for (const TileShape &t : kTileShapes) {
    if (t.tile != form) continue;
    const bool one_round = tile_count(M, N, t.bm, t.bn, batch) <= cus;
    if (form == MfmaTile::T64) {
      c.ksplit = one_round && K >= 512;
      c.long_k = c.ksplit && K >= 1280;
    } else if (form == MfmaTile::T32x64 || form == MfmaTile::T32) {
      c.long_k = one_round;
    }
  }
  return c;
}

// Measured on 256 CUs (kernel trace and HIP events): 1000 x 1500 x 777
// takes 64 x 96 (256 tiles, one 12-wave work-group per CU: 24.9 us, against
// 25.4 for 32 x 64 -- 768 tiles, three work-groups per CU -- and 31.9 for
// 64 x 64, whose 384 tiles leave half the CUs idle in the second round);
// 1024^3 takes 64 x 64 (256 tiles); 2048^3 128 x 128; 8192^3 256 x 256;
// 512^3 and 1000 x 130 x 2048 take 32 x 32; 256^3 16 x 16.
//
// The 16 x 16 small-product tile, measured on 256 CUs against the best
// buffer-to-LDS tile (kernel trace): 256^3 4.33 -> 3.74 us, 256 x 256 x 1024
// 7.46 -> 6.61, 128^3 3.88 -> 3.09, 256^2 x 32 3.70 -> 2.92 (its tiles read
// 4-32 KiB per CU, or 128 KiB where the 32 x 32 tile fills a quarter of the
// CUs), even on 512 x 512 x 64 (32 KiB) and 100 x 3000 x 64 (41 KiB).  At 50
// KiB per CU it loses (640 x 640 x 64: 4.38-4.81 against 4.11-4.60 over
// three sweeps), and where its tiles read 64-100 KiB per CU and a
// buffer-to-LDS tile keeps at least half the matrix-core time on C it loses
// more (384 x 384 x 256: 5.48 against 4.65; 768 x 256 x 256: 5.28 against
// 4.52; 512 x 512 x 128: 4.31 against 4.03; 640 x 640 x 128: 5.52 against
// 4.64), and past 128 KiB per CU by more still (384 x 384 x 512: 7.81
// against 5.71; 1000 x 130 x 1024: 16.06 against 8.79).  Shapes with more
// than 8 of its tiles per CU were not measured.
TileChoice choose_mfma_tile(long M, long N, long K, int cus, long batch) {
  auto eff = [&](const TileShape &t) {
    if (t.tile == MfmaTile::T16) return 0.0;
    // One 64 x 96 work-group (12 waves) fills a CU, so a second round could
    // not overlap the first one's slices: one round only.
    if (t.tile == MfmaTile::T64x96 && tile_count(M, N, t.bm, t.bn, batch) > cus) return 0.0;
    return tile_efficiency(t, M, N, cus, batch);
  };
  double best = 0.0;
  for (const TileShape &t : kTileShapes) best = fmax(best, eff(t));
  if (small_product(M, N, K, cus, batch) &&
      (small_bytes_per_cu(M, N, K, cus, batch) <= 48.0 * 1024 || best < 0.5))
    return with_slice_rule(MfmaTile::T16, M, N, K, cus, batch);
  for (const TileShape &t : kTileShapes)
    if (best > 0.0 && eff(t) >= 0.97 * best) return with_slice_rule(t.tile, M, N, K, cus, batch);
  return with_slice_rule(MfmaTile::T128, M, N, K, cus, batch);
}

TileGeometry tile_geometry(TileChoice tile, bool wide, long K) {
  if (tile.tile == MfmaTile::T16) {
    int ng = 1;  // groups of 16 k per wave and pass, as mfma_small.hip picks them
    while (ng < 16 && 64L * ng < K) ng *= 2;
    return {16, 16, 64 * ng, 4};
  }
  const DmaGeom g = dma_geom(dma_cfg(tile, wide));
  return {g.bm, g.bn, g.bk, g.ksets};
}

// Load widths of the buffer-to-LDS kernel for configuration c and depth K.
// The 64 x 96 tile (12 waves, three per SIMD) keeps 16-byte loads to
// operands that the stricter rule of the other kernels admits (w.a16,
// w.b16): with 16-byte A loads wherever the rule of the buffer-to-LDS
// kernel allows them it ran slower than with 4-byte loads on most shapes
// measured (HIP events, three alternations on one box: 1000 x 1500 x 1199
// 33.6 against 31.7 us, 960 x 1600 x 777 22.9 against 21.9), while the
// other tiles gained (512 x 512 x 1199 8.8 against 10.4 us, 800 x 1280 x
// 1199 22.5 against 24.9, 2048 x 2048 x 2047 118.6 against 125.4).  With a
// ragged K (the partial slice computed first) it also takes 4-byte loads
// from K = 960 on, where they beat 16-byte loads from 16-byte aligned
// operands (1000 x 1500 x K, two sweeps: K = 1000 26.6 against 27.9 us,
// 1200 30.8 against 33.4, 2000 48.0-48.9 against 52.7; 1200 x 1200 x 1200
// 31.6 against 33.0), as they do not at shorter K (700 20.0-20.4 against
// 19.3-19.7, 784 21.9-22.1 against 21.2-21.4) nor with K a multiple of 32
// (1600: 43.7 against 42.7).
static void dma_widths(DmaCfg c, LoadWidths w, long K, bool &va, bool &vb) {
  if (c == DmaCfg::C64x96) {
    const bool wide = K % 32 == 0 || K < 960;
    va = wide && w.a16;
    vb = wide && w.b16;
  } else {
    va = w.a_dma;
    vb = w.b_dma;
  }
}

hipError_t launch_mfma(TileChoice tile, MfmaPath path, const GemmArgs &p, LoadWidths w,
                       hipStream_t stream) {
  if (path == MfmaPath::Staged) return launch_staged(tile.tile, true, p, w.a16, w.b16, stream);
  if (tile.tile == MfmaTile::T16 && path != MfmaPath::Unpadded)
    return launch_small(p, false, false, w.a16, w.b16, stream);
  const DmaCfg c = dma_cfg(tile, w.a_dma && w.b_dma);
  const DmaGeom g = dma_geom(c);
  // A slice whose offsets pass a buffer descriptor's 32-bit range takes the
  // register-staged kernel (64-bit addressing).
  if (!dma_offsets_fit(g.bm, p.lda, g.bk, p.ldb)) {
    if (path == MfmaPath::Serial) return hipErrorInvalidValue;
    return launch_staged(tile.tile, path != MfmaPath::Unpadded, p, w.a16, w.b16, stream);
  }
  bool va, vb;
  dma_widths(c, w, p.K, va, vb);
  if (path == MfmaPath::Serial)
    return launch_dma_layout<false, false, true, false, 2>(c, p, va, vb, stream);
  if (path == MfmaPath::Unpadded) return launch_dma_layout<false, false, false>(c, p, va, vb, stream);
  return launch_dma_layout<false, false, true>(c, p, va, vb, stream);
}

hipError_t launch_mfma_phases(TileChoice tile, const GemmArgs &p, LoadWidths w, long *workgroups,
                              hipStream_t stream) {
  if (tile.tile == MfmaTile::T16) {
    *workgroups = small_workgroups(p.M, p.N, 1);
    return p.phases == nullptr ? hipSuccess : launch_small_phases(p, w.a16, stream);
  }
  const DmaCfg c = dma_cfg(tile, w.a_dma && w.b_dma);
  const DmaGeom g = dma_geom(c);
  if (!dma_offsets_fit(g.bm, p.lda, g.bk, p.ldb)) return hipErrorInvalidValue;
  *workgroups = (long)((p.M + g.bm - 1) / g.bm) * ((p.N + g.bn - 1) / g.bn);
  if (p.phases == nullptr) return hipSuccess;
  bool va, vb;
  dma_widths(c, w, p.K, va, vb);
  return launch_dma_layout<false, false, true, true>(c, p, va, vb, stream);
}

hipError_t launch_mfma_general(TileChoice tile, const GemmArgs &p, bool ta, bool tb, LoadWidths w,
                               hipStream_t stream) {
  if (tile.tile == MfmaTile::T16) return launch_small(p, ta, tb, w.a16, w.b16, stream);
  const DmaCfg c = dma_cfg(tile, !ta && !tb && w.a_dma && w.b_dma);
  bool va, vb;
  dma_widths(c, w, p.K, va, vb);
  const DmaGeom g = dma_geom(c);
  if (!dma_offsets_fit(ta ? g.bk : g.bm, p.lda, tb ? g.bn : g.bk, p.ldb))
    return hipErrorInvalidValue;
  if (!ta && !tb) return launch_dma_layout<false, false, true>(c, p, va, vb, stream);
  if (!ta) return launch_dma_layout<false, true, true>(c, p, va, vb, stream);
  if (!tb) return launch_dma_layout<true, false, true>(c, p, va, vb, stream);
  return launch_dma_layout<true, true, true>(c, p, va, vb, stream);
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
