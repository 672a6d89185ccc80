// noalloc.hip -- sgemm_run_bf16x3_ex_noalloc: the bfloat16-split product for
// callers that cannot allocate device memory, with its split planes in a
// library-held buffer instead of a caller's workspace.
//
// `scratch` is a file-scope device array: every GPU the library runs this
// entry point on holds its own copy, allocated by the runtime when this
// file's code object is loaded on that device, until the process ends.  In
// host code the name `scratch` is only a host-side stand-in, not a device
// address, so it is never passed to a kernel or a copy: the device address is
// looked up once per device (with that device current) by hipGetSymbolAddress
// and kept in g_addr, and only that address is used.  The lookup happens at
// the entry point's first call on a device rather than in sgemm_create, so a
// process that never calls this entry point never loads the 64 MiB array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "api_internal.hpp"
#include "sgemm.h"
#include "sgemm_bf16x3.h"

static __device__ __align__(256) unsigned char scratch[SGEMM_BF16X3_NOALLOC_MAX_BYTES];

namespace {

constexpr int64_t kScratchBytes = SGEMM_BF16X3_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
std::atomic<void *> g_addr[kMaxDevices];  // device address of `scratch`, per device

// This device's address of `scratch` (looked up on first use, then cached).
int scratch_address(void **out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return SGEMM_ERR_HIP;
  if (d < 0 || d >= kMaxDevices) return SGEMM_ERR_UNSUPPORTED_DEVICE;
  void *p = g_addr[d].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_addr[d].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return SGEMM_ERR_HIP;
      g_addr[d].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SGEMM_OK;
}

}  // namespace

extern "C" int sgemm_run_bf16x3_ex_noalloc(int transA, int transB, int64_t M, int64_t N,
                                           int64_t K, float alpha, const float *A, int64_t lda,
                                           const float *B, int64_t ldb, float beta, float *C,
                                           int64_t ldc, void *stream) {
  int64_t need = 0;
  const int chk =
      sgemm_api::bf16x3_ex_check(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, &need);
  if (chk != SGEMM_OK) return chk;
  if (need > kScratchBytes) return SGEMM_ERR_TOO_LARGE;
  if (!sgemm_api::ready()) return SGEMM_ERR_NOT_INITIALIZED;
  void *ws = nullptr;
  if (need > 0) {
    const int rc = scratch_address(&ws);
    if (rc != SGEMM_OK) return rc;
  }
  // The split kernel writes every byte of the planes it uses, padding
  // included, so nothing left by an earlier call needs clearing.
  return sgemm_run_bf16x3_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ws,
                             need > 0 ? kScratchBytes : 0, stream);
}
