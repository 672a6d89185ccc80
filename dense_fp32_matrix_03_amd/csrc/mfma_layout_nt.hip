// mfma_layout_nt.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: A as stored, B stored transposed.
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<false, true, true, false>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
