// vector_add.hip -- C[i] = A[i] + B[i] over n floats (blog "【infra之路】03_动手写
// CUDA Kernel", 实验 1, vector addition: one add per element, effective
// bandwidth counted as three arrays of n floats per call).
//
// On MI355X this is pure HBM streaming.  Each thread adds one 16-byte chunk
// (four floats) of A and B, read with non-temporal loads: the operands are
// used once, so they should not displace other data from the caches, and
// measured over 2^24 and 2^28 floats this shape beat 2, 4 or 8 chunks per
// thread, grid-stride loops, 512- and 1024-thread groups and non-temporal
// stores (6.4 - 6.9 TB/s against 5.7 - 6.1 for plain loads, on zero-filled
// arrays; non-zero data streams about 9% slower).  If any of A,
// B, C is not 16-byte aligned, a one-float-per-lane kernel (four floats per
// thread, strided by the group size) runs instead.  Each element is read and
// written by one thread, loads before the store, so C may be A or B itself.
// The adds are plain single precision (round to nearest even), never packed.
#include "common.hpp"
#include "dispatch.hpp"

namespace sgemm {

constexpr int kVaddThreads = 256;
constexpr int kVaddUnroll1 = 4;  // floats per thread in the unaligned kernel

// Chunk c of the 16-byte view covers floats 4c .. 4c+3.  The n % 4 tail is
// added by the first threads of the last work-group.
__global__ void __launch_bounds__(kVaddThreads)
vector_add_x4_kernel(const f32x4 *A, const f32x4 *B, f32x4 *C, long chunks, const float *At,
                     const float *Bt, float *Ct, int tail) {
  const long c = (long)blockIdx.x * kVaddThreads + threadIdx.x;
  if (c < chunks) {
    const f32x4 a = __builtin_nontemporal_load(A + c);
    const f32x4 b = __builtin_nontemporal_load(B + c);
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = a[e] + b[e];
    C[c] = r;
  }
  if (blockIdx.x == gridDim.x - 1 && (int)threadIdx.x < tail)
    Ct[threadIdx.x] = At[threadIdx.x] + Bt[threadIdx.x];
}

__global__ void __launch_bounds__(kVaddThreads)
vector_add_x1_kernel(const float *A, const float *B, float *C, long n) {
  const long base = (long)blockIdx.x * (kVaddThreads * kVaddUnroll1) + threadIdx.x;
  float a[kVaddUnroll1], b[kVaddUnroll1];
#pragma unroll
  for (int u = 0; u < kVaddUnroll1; ++u) {
    const long i = base + (long)u * kVaddThreads;
    if (i < n) {
      a[u] = __builtin_nontemporal_load(A + i);
      b[u] = __builtin_nontemporal_load(B + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kVaddUnroll1; ++u) {
    const long i = base + (long)u * kVaddThreads;
    if (i < n) C[i] = a[u] + b[u];
  }
}

hipError_t launch_vector_add(long n, const float *A, const float *B, float *C,
                             hipStream_t stream) {
  const bool wide = ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
                      reinterpret_cast<uintptr_t>(C)) & 15u) == 0;
  if (wide) {
    const long chunks = n / 4;
    const int tail = (int)(n % 4);
    long blocks = (chunks + kVaddThreads - 1) / kVaddThreads;
    if (blocks < 1) blocks = 1;  // the tail alone still needs a work-group
    hipLaunchKernelGGL(vector_add_x4_kernel, dim3((unsigned)blocks), dim3(kVaddThreads), 0,
                       stream, reinterpret_cast<const f32x4 *>(A),
                       reinterpret_cast<const f32x4 *>(B), reinterpret_cast<f32x4 *>(C), chunks,
                       A + 4 * chunks, B + 4 * chunks, C + 4 * chunks, tail);
  } else {
    constexpr long per_block = (long)kVaddThreads * kVaddUnroll1;
    const long blocks = (n + per_block - 1) / per_block;
    hipLaunchKernelGGL(vector_add_x1_kernel, dim3((unsigned)blocks), dim3(kVaddThreads), 0,
                       stream, A, B, C, n);
  }
  return hipGetLastError();
}

}  // namespace sgemm
