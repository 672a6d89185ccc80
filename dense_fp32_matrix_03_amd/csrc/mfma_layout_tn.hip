// mfma_layout_tn.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A stored transposed, B as stored.
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<true, false, true, false>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
