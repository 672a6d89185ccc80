// mfma_layout_nn_serial.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A and B as stored, in the race-triage schedule (no load in
// flight while a slice is computed; SGEMM_VARIANT_MFMA_SERIAL).
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<false, false, true, false, 2>(DmaCfg, const GemmArgs &,
                                                                    bool, bool, hipStream_t);
}  // namespace sgemm
