// mfma_layout_nn_phases.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A and B as stored, with per-work-group phase timestamps (sgemm_phase_times).
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<false, false, true, true>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
