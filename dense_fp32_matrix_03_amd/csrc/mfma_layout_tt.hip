// mfma_layout_tt.hip -- the buffer-to-LDS configurations of mfma_configs.hpp
// for one operand layout: both operands stored transposed.
#include "mfma_configs.hpp"

namespace sgemm {
template hipError_t launch_dma_layout<true, true, true, false>(DmaCfg, const GemmArgs &, bool, bool,
                                                     hipStream_t);
}  // namespace sgemm
