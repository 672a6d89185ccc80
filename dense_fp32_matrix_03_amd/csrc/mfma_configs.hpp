// mfma_configs.hpp -- the block-tile configurations of the buffer-to-LDS
// matrix-core kernel that the library instantiates, and one launcher per
// operand layout.  Each layout (and the unswizzled plain layout kept for the
// ablation) is instantiated in a translation unit of its own
// (mfma_layout_*.hip), so that the library builds in parallel.
#pragma once

#include "dispatch.hpp"
#include "mfma_dma.hpp"

namespace sgemm {

// Configurations: block tile BM x BN, K slice BK, a WM x WN grid of waves per
// k set and KSPLIT k sets.  Every configuration walks K in the same order
// for every operand layout, so stored transposes give the plain layout's bits.
//   C256     256 x 256 x 32, 2 x 4 waves of 128 x 64 (plain layout, 16-byte loads)
//   C128     128 x 128 x 32, 4 x 2 waves of  32 x 64
//   C64       64 x  64 x 32, 2 x 2 waves of  32 x 32 (4 waves)
//   C64K2     the same with two k sets (8 waves)
//   C64K2L    C64K2 with 64-float K slices
//   C64x96    64 x  96 x 32, 2 x 3 waves of  32 x 32, two k sets (12 waves)
//   C32x64    32 x  64 x 32, 1 x 2 waves of  32 x 32, two k sets (4 waves)
//   C32x64L   the same with 64-float K slices
//   C32       32 x  32 x 32, one wave, four k sets (4 waves)
//   C32L      the same with 64-float K slices
enum class DmaCfg { C256, C128, C64, C64K2, C64K2L, C64x96, C32x64, C32x64L, C32, C32L };

// Block tile, K slice and k sets (the KSPLIT of launch_dma_layout below).
struct DmaGeom {
  int bm, bn, bk, ksets;
};

inline DmaGeom dma_geom(DmaCfg c) {
  switch (c) {
    case DmaCfg::C256: return {256, 256, 32, 1};
    case DmaCfg::C128: return {128, 128, 32, 1};
    case DmaCfg::C64: return {64, 64, 32, 1};
    case DmaCfg::C64K2: return {64, 64, 32, 2};
    case DmaCfg::C64K2L: return {64, 64, 64, 2};
    case DmaCfg::C64x96: return {64, 96, 32, 2};
    case DmaCfg::C32x64: return {32, 64, 32, 2};
    case DmaCfg::C32x64L: return {32, 64, 64, 2};
    case DmaCfg::C32: return {32, 32, 32, 4};
    case DmaCfg::C32L: return {32, 32, 64, 4};
  }
  return {0, 0, 0, 0};
}

// Launch configuration c for operand layout (TA, TB); SWZ = false drops the
// LDS swizzle; PHASES selects the diagnostic instantiation that writes
// per-work-group timestamps to p.phases; SCHED = 2 the race-triage schedule
// (no load in flight while a slice is computed; same bits).  C256 is instantiated only for the
// plain layout with 16-byte loads on both operands (its other forms would
// spill); asked for anything else it returns hipErrorInvalidValue.
template <bool TA, bool TB, bool SWZ, bool PHASES = false, int SCHED = 1>
hipError_t launch_dma_layout(DmaCfg c, const GemmArgs &p, bool va, bool vb, hipStream_t s);

template <bool TA, bool TB, bool SWZ, bool PHASES, int SCHED>
hipError_t launch_dma_layout(DmaCfg c, const GemmArgs &p, bool va, bool vb, hipStream_t s) {
  constexpr int kGroupM = 8;  // tile rows per raster group
  switch (c) {
    case DmaCfg::C256:
      if constexpr (!TA && !TB) {
        if (!(va && vb)) return hipErrorInvalidValue;
        launch_dma_kernel<256, 256, 32, 2, 4, SWZ, SCHED, true, true, false, false, 1, 2, PHASES>(
            p, s, kGroupM);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    case DmaCfg::C128:
      launch_dma_widths<128, 128, 32, 4, 2, SWZ, SCHED, TA, TB, 1, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C64:
      launch_dma_widths<64, 64, 32, 2, 2, SWZ, SCHED, TA, TB, 1, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C64K2:
      launch_dma_widths<64, 64, 32, 2, 2, SWZ, SCHED, TA, TB, 2, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C64K2L:
      launch_dma_widths<64, 64, 64, 2, 2, SWZ, SCHED, TA, TB, 2, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C64x96:
      launch_dma_widths<64, 96, 32, 2, 3, SWZ, SCHED, TA, TB, 2, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C32x64:
      launch_dma_widths<32, 64, 32, 1, 2, SWZ, SCHED, TA, TB, 2, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C32x64L:
      launch_dma_widths<32, 64, 64, 1, 2, SWZ, SCHED, TA, TB, 2, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C32:
      launch_dma_widths<32, 32, 32, 1, 1, SWZ, SCHED, TA, TB, 4, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
    case DmaCfg::C32L:
      launch_dma_widths<32, 32, 64, 1, 1, SWZ, SCHED, TA, TB, 4, 2,
                        PHASES>(p, va, vb, s, kGroupM);
      break;
  }
  return hipGetLastError();
}

// Instantiated in mfma_layout_*.hip.
extern template hipError_t launch_dma_layout<false, false, true, false>(DmaCfg, const GemmArgs &,
                                                                        bool, bool, hipStream_t);
extern template hipError_t launch_dma_layout<false, false, false, false>(DmaCfg,
                                                                         const GemmArgs &, bool,
                                                                         bool, hipStream_t);
extern template hipError_t launch_dma_layout<false, true, true, false>(DmaCfg, const GemmArgs &,
                                                                       bool, bool, hipStream_t);
extern template hipError_t launch_dma_layout<true, false, true, false>(DmaCfg, const GemmArgs &,
                                                                       bool, bool, hipStream_t);
extern template hipError_t launch_dma_layout<true, true, true, false>(DmaCfg, const GemmArgs &,
                                                                      bool, bool, hipStream_t);
extern template hipError_t launch_dma_layout<false, false, true, true>(DmaCfg, const GemmArgs &,
                                                                       bool, bool, hipStream_t);
extern template hipError_t launch_dma_layout<false, false, true, false, 2>(DmaCfg,
                                                                          const GemmArgs &, bool,
                                                                          bool, hipStream_t);

}  // namespace sgemm
