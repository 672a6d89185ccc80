// ceiling.hip -- the attainable matrix-core rate: a register-only loop of
// independent accumulator chains on every compute unit, no memory traffic.
// The product kernels' rates are reported against it beside the published
// peak.  Four 256-thread work-groups per CU (four waves per SIMD), eight
// chains per wave, so no chain waits on its own previous result.
#include "common.hpp"
#include "dispatch.hpp"

namespace sgemm {

typedef __bf16 ceiling_bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kCeilChains = 8;
constexpr int kCeilThreads = 256;
constexpr int kCeilBlocksPerCu = 4;

template <int WHICH>
__global__ void __launch_bounds__(kCeilThreads) mfma_ceiling_kernel(float *out, int iters) {
  f32x16 acc[kCeilChains];
#pragma unroll
  for (int j = 0; j < kCeilChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const float a = 1.0f + threadIdx.x * 1e-7f, b = 1.0f - threadIdx.x * 1e-7f;
  if constexpr (WHICH == 0) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kCeilChains; ++j) acc[j] = mfma32x32x2(a, b, acc[j]);
    }
  } else {
    ceiling_bf16x8 va, vb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      va[e] = (__bf16)a;
      vb[e] = (__bf16)b;
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kCeilChains; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCeilChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(long)blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

long mfma_ceiling_outputs(int cus) { return (long)cus * kCeilBlocksPerCu * kCeilThreads; }

hipError_t launch_mfma_ceiling(int which, int iters, float *out, int cus, double *flops,
                               hipStream_t stream) {
  const int blocks = cus * kCeilBlocksPerCu;
  const double per_instr = which == 0 ? 2.0 * 32 * 32 * 2 : 2.0 * 32 * 32 * 16;
  *flops = per_instr * kCeilChains * (double)iters * blocks * (kCeilThreads / kWave);
  if (which == 0)
    hipLaunchKernelGGL(mfma_ceiling_kernel<0>, dim3(blocks), dim3(kCeilThreads), 0, stream, out,
                       iters);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<1>, dim3(blocks), dim3(kCeilThreads), 0, stream, out,
                       iters);
  return hipGetLastError();
}

}  // namespace sgemm
