// mfma_layout_nn.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A and B as stored (the plain product and the general form without transposes).
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<false, false, true, false>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
