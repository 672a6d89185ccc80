// mfma_staged.hip -- the register-staged matrix-core kernel (mfma_gemm.hpp):
// the ablation SGEMM_VARIANT_MFMA_STAGED, and sgemm_run's fallback when a
// leading dimension puts one K slice beyond a buffer descriptor's 32-bit
// offsets.  It has no k split, so the 64 x 96, 32 x 64 and 32 x 32 tiles run
// on its 64 x 64 tile.
#include "dispatch.hpp"
#include "mfma_gemm.hpp"

namespace sgemm {

hipError_t launch_staged(MfmaTile tile, bool padded, const GemmArgs &p, bool va, bool vb,
                         hipStream_t stream) {
  constexpr int kStoreGroup = 1;  // write the next slice to LDS after group 1 of 4
  if (tile == MfmaTile::T256 && !(va && vb)) tile = MfmaTile::T128;  // 4-byte forms would spill
  switch (tile) {
    case MfmaTile::T256:
      return padded ? launch_staged_cfg<256, 256, 32, 2, 4, 4, kStoreGroup>(p, va, vb, stream)
                    : launch_staged_cfg<256, 256, 32, 2, 4, 0, kStoreGroup>(p, va, vb, stream);
    case MfmaTile::T128:
      return padded ? launch_staged_cfg<128, 128, 32, 2, 2, 4, kStoreGroup>(p, va, vb, stream)
                    : launch_staged_cfg<128, 128, 32, 2, 2, 0, kStoreGroup>(p, va, vb, stream);
    default:
      return padded ? launch_staged_cfg<64, 64, 32, 2, 2, 4, kStoreGroup>(p, va, vb, stream)
                    : launch_staged_cfg<64, 64, 32, 2, 2, 0, kStoreGroup>(p, va, vb, stream);
  }
}

}  // namespace sgemm
