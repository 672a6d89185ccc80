// mfma_layout_nn_unswizzled.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A and B as stored, without the LDS swizzle (SGEMM_VARIANT_MFMA_UNPADDED).
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<false, false, false, false>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
