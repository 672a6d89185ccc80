// api.hip -- the C interface declared in include/sgemm.h,
// include/sgemm_bf16x3.h and include/vector_add.h: argument checks, device
// check, and the choice of kernel configuration for each call.
#include <stdint.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "api_internal.hpp"
#include "dispatch.hpp"
#include "sgemm.h"
#include "sgemm_bf16x3.h"
#include "vector_add.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
  bool supported = false;
  int cus = 0;
};

// One cached entry per device: `known` is set (release) after `info` is
// filled, so a call that sees it set reads `info` without the lock.
struct DeviceSlot {
  std::atomic<bool> known{false};
  DeviceInfo info;
};

std::mutex g_mu;
int g_refs = 0;
std::atomic<int> g_ready{0};
DeviceSlot g_dev[kMaxDevices];

// Query (once) and cache what the dispatcher needs to know about device d.
int device_info(int d, DeviceInfo *out) {
  if (d < 0 || d >= kMaxDevices) return SGEMM_ERR_UNSUPPORTED_DEVICE;
  DeviceSlot &slot = g_dev[d];
  if (!slot.known.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!slot.known.load(std::memory_order_relaxed)) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, d) != hipSuccess) return SGEMM_ERR_HIP;
      slot.info.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
      slot.info.cus = prop.multiProcessorCount;
      slot.known.store(true, std::memory_order_release);
    }
  }
  *out = slot.info;
  return out->supported ? SGEMM_OK : SGEMM_ERR_UNSUPPORTED_DEVICE;
}

int current_device_info(DeviceInfo *out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return SGEMM_ERR_HIP;
  return device_info(d, out);
}

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// A launch's work-items (work-groups x threads) must fit 32 bits.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
// bfloat16-split product: K up to 2^21 keeps a 256-row slice of a plane
// within a buffer descriptor's range; (M + N) * Kp up to 2^34 keeps the split
// launches below 2^32 work-items.
constexpr int64_t kMaxBf16x3K = int64_t(1) << 21;
constexpr int64_t kMaxBf16x3Split = int64_t(1) << 34;

// Whether `batch` products of M x N, one `threads`-wide work-group per
// bm x bn block of C, fit one launch.  sgemm_run and the general form pick a
// tile whose launch fits (the 128 x 128 tile, 128 threads per 64 x 64 block,
// always does once 256 per 64 x 64 block fit); the vector-FMA rungs use 256
// threads per 16 x 16 block (or the equivalent).
bool grid_fits(int64_t M, int64_t N, int64_t batch, int64_t bm, int64_t bn, int64_t threads) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  return batch == 0 || tiles <= kMaxWorkItems / threads / batch;
}

// Shared argument checks of every product entry point.
int check_args(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
               int64_t ldb, const float *C, int64_t ldc) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_INVALID_VALUE;
  if (lda < (K > 1 ? K : 1) || ldb < (N > 1 ? N : 1) || ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_ERR_TOO_LARGE;
  if (!grid_fits(M, N, 1, 64, 64, 256)) return SGEMM_ERR_TOO_LARGE;
  if (M == 0 || N == 0) return SGEMM_OK;
  if (!C) return SGEMM_ERR_INVALID_VALUE;
  if (K > 0 && (!A || !B)) return SGEMM_ERR_INVALID_VALUE;
  return SGEMM_OK;
}

inline bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
inline bool aligned4(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

// Which operands take 16-byte loads (sgemm::LoadWidths).  The small-product
// and register-staged kernels load 16-byte aligned chunks: the base, the
// leading dimension, the batch stride and the stored width must allow that.
// The buffer-to-LDS kernel loads 16-byte chunks from any dword-aligned
// address (its partial last K slice takes 4-byte loads where a chunk would
// reach past K), so it needs a stored width that is a multiple of 4 only
// where the chunks run along m or n: A stored transposed, B as given.
sgemm::LoadWidths load_widths(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const float *A,
                              int64_t lda, int64_t strideA, const float *B, int64_t ldb,
                              int64_t strideB) {
  const int64_t a_cols = ta ? M : K, b_cols = tb ? K : N;
  sgemm::LoadWidths w;
  w.a16 = aligned16(A) && lda % 4 == 0 && strideA % 4 == 0 && a_cols % 4 == 0;
  w.b16 = aligned16(B) && ldb % 4 == 0 && strideB % 4 == 0 && b_cols % 4 == 0;
  w.a_dma = aligned4(A) && (!ta || M % 4 == 0);
  w.b_dma = aligned4(B) && (tb || N % 4 == 0);
  return w;
}

}  // namespace

extern "C" {

int sgemm_create(void) {
  DeviceInfo di;
  const int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  std::lock_guard<std::mutex> lk(g_mu);
  ++g_refs;
  g_ready.store(1, std::memory_order_release);
  return SGEMM_OK;
}

int sgemm_destroy(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_refs == 0) return SGEMM_ERR_NOT_INITIALIZED;
  if (--g_refs == 0) g_ready.store(0, std::memory_order_release);
  return SGEMM_OK;
}

int sgemm_run_variant(int variant, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, void *stream) {
  // Argument errors are reported before anything touches the runtime.
  if (variant < 0 || variant >= SGEMM_NUM_VARIANTS) return SGEMM_ERR_INVALID_VALUE;
  int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != SGEMM_OK) return rc;
  if (variant <= SGEMM_VARIANT_DBUF && !grid_fits(M, N, 1, 16, 16, 256)) return SGEMM_ERR_TOO_LARGE;
  // Forced tiles: 512 threads per 64 x 64 block, 768 per 64 x 96, 256 per
  // 32 x 64, 32 x 32 or 16 x 16 block (sgemm_run only picks a tile whose
  // launch fits).
  if (variant == SGEMM_VARIANT_MFMA_64 && !grid_fits(M, N, 1, 64, 64, 512))
    return SGEMM_ERR_TOO_LARGE;
  if (variant == SGEMM_VARIANT_MFMA_64X96 && !grid_fits(M, N, 1, 64, 96, 768))
    return SGEMM_ERR_TOO_LARGE;
  if (variant == SGEMM_VARIANT_MFMA_32X64 && !grid_fits(M, N, 1, 32, 64, 256))
    return SGEMM_ERR_TOO_LARGE;
  if (variant == SGEMM_VARIANT_MFMA_32 && !grid_fits(M, N, 1, 32, 32, 256))
    return SGEMM_ERR_TOO_LARGE;
  if (variant == SGEMM_VARIANT_MFMA_16 && !grid_fits(M, N, 1, 16, 16, 256))
    return SGEMM_ERR_TOO_LARGE;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  if (M == 0 || N == 0) return SGEMM_OK;
  DeviceInfo di;
  rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;

  sgemm::GemmArgs p;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t err;
  if (K == 0) {
    err = sgemm::launch_scale(p, s);  // beta = 0: zeros
  } else {
    const sgemm::LoadWidths w = load_widths(false, false, M, N, K, A, lda, 0, B, ldb, 0);
    using sgemm::MfmaPath;
    using sgemm::MfmaTile;
    const sgemm::TileChoice autotile = sgemm::choose_mfma_tile(M, N, K, di.cus);
    // A forced tile keeps the K-slice rule of the automatic choice, so it
    // gives sgemm_run's bits whenever sgemm_run picks the same tile.
    auto forced = [&](MfmaTile t) { return sgemm::with_slice_rule(t, M, N, K, di.cus); };
    switch (variant) {
      case SGEMM_VARIANT_NAIVE:
      case SGEMM_VARIANT_LDS:
      case SGEMM_VARIANT_REG:
      case SGEMM_VARIANT_DBUF:
        err = sgemm::launch_valu(variant - SGEMM_VARIANT_NAIVE, p, w.a16, w.b16, s);
        break;
      case SGEMM_VARIANT_MFMA_256:
        err = sgemm::launch_mfma(forced(MfmaTile::T256), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_128:
        err = sgemm::launch_mfma(forced(MfmaTile::T128), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_64:
        err = sgemm::launch_mfma(forced(MfmaTile::T64), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_64X96:
        err = sgemm::launch_mfma(forced(MfmaTile::T64x96), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_32X64:
        err = sgemm::launch_mfma(forced(MfmaTile::T32x64), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_32:
        err = sgemm::launch_mfma(forced(MfmaTile::T32), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_16:
        err = sgemm::launch_mfma(forced(MfmaTile::T16), MfmaPath::Auto, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_STAGED:
        err = sgemm::launch_mfma(autotile, MfmaPath::Staged, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_UNPADDED:
        err = sgemm::launch_mfma(autotile, MfmaPath::Unpadded, p, w, s);
        break;
      case SGEMM_VARIANT_MFMA_DWORD:
        // 4-byte loads for both operands whatever their alignment.
        err = sgemm::launch_mfma(autotile, MfmaPath::Auto, p, sgemm::LoadWidths{}, s);
        break;
      case SGEMM_VARIANT_MFMA_SERIAL:
        err = sgemm::launch_mfma(autotile, MfmaPath::Serial, p, w, s);
        if (err == hipErrorInvalidValue) return SGEMM_ERR_TOO_LARGE;  // no register-staged form
        break;
      default:
        err = sgemm::launch_mfma(autotile, MfmaPath::Auto, p, w, s);
        break;
    }
  }
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_run(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
              int64_t ldb, float *C, int64_t ldc, void *stream) {
  return sgemm_run_variant(SGEMM_VARIANT_MFMA, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int sgemm_tile_choice(int64_t M, int64_t N, int64_t K, int64_t batch, int cus, int *bm, int *bn,
                      int *bk, int *ksets) {
  if (M < 1 || N < 1 || K < 1 || batch < 1 || cus < 1) return SGEMM_ERR_INVALID_VALUE;
  if (!bm || !bn || !bk || !ksets) return SGEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim) return SGEMM_ERR_TOO_LARGE;
  if (!grid_fits(M, N, batch, 64, 64, 256)) return SGEMM_ERR_TOO_LARGE;
  const sgemm::TileChoice t = sgemm::choose_mfma_tile(M, N, K, cus, batch);
  const sgemm::TileGeometry g = sgemm::tile_geometry(t, true, K);
  *bm = g.bm;
  *bn = g.bn;
  *bk = g.bk;
  *ksets = g.ksets;
  return SGEMM_OK;
}

int sgemm_phase_times(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, uint64_t *times,
                      int64_t times_len, int64_t *workgroups, void *stream) {
  if (!workgroups || M < 1 || N < 1 || K < 1) return SGEMM_ERR_INVALID_VALUE;
  int rc = check_args(M, N, K, A, lda, B, ldb, C, ldc);
  if (rc != SGEMM_OK) return rc;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  DeviceInfo di;
  rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  sgemm::GemmArgs p;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  const sgemm::LoadWidths w = load_widths(false, false, M, N, K, A, lda, 0, B, ldb, 0);
  const sgemm::TileChoice tile = sgemm::choose_mfma_tile(M, N, K, di.cus);
  long wgs = 0;
  hipError_t err = sgemm::launch_mfma_phases(tile, p, w, &wgs, nullptr);  // count only
  if (err == hipErrorInvalidValue) return SGEMM_ERR_TOO_LARGE;
  *workgroups = wgs;
  if (times == nullptr) return SGEMM_OK;
  if (times_len < 8 * (int64_t)wgs) return SGEMM_ERR_INVALID_VALUE;
  p.phases = reinterpret_cast<unsigned long long *>(times);
  err = sgemm::launch_mfma_phases(tile, p, w, &wgs, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_run_strided_batched(int transA, int transB, int64_t M, int64_t N, int64_t K,
                              float alpha, const float *A, int64_t lda, int64_t strideA,
                              const float *B, int64_t ldb, int64_t strideB, float beta,
                              float *C, int64_t ldc, int64_t strideC, int64_t batch,
                              void *stream) {
  if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return SGEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0 || batch < 0) return SGEMM_ERR_INVALID_VALUE;
  if (strideA < 0 || strideB < 0 || strideC < 0) return SGEMM_ERR_INVALID_VALUE;
  // Distinct products write disjoint C matrices.
  if (batch > 1 && M > 0 && N > 0 && (__int128)(M - 1) * ldc + N > strideC)
    return SGEMM_ERR_INVALID_VALUE;
  const int64_t a_cols = transA ? M : K, b_cols = transB ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || batch > kMaxDim) return SGEMM_ERR_TOO_LARGE;
  if (!grid_fits(M, N, batch, 64, 64, 256)) return SGEMM_ERR_TOO_LARGE;
  const bool reads_ab = K > 0 && alpha != 0.f;
  if (M > 0 && N > 0 && batch > 0) {
    if (!C) return SGEMM_ERR_INVALID_VALUE;
    if (reads_ab && (!A || !B)) return SGEMM_ERR_INVALID_VALUE;
  }
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  if (M == 0 || N == 0 || batch == 0) return SGEMM_OK;
  DeviceInfo di;
  int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;

  sgemm::GemmArgs p;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  p.alpha = alpha;
  p.beta = beta;
  p.strideA = strideA;
  p.strideB = strideB;
  p.strideC = strideC;
  p.batch = (int)batch;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t err;
  if (!reads_ab) {
    err = sgemm::launch_scale(p, s);  // C = beta C (zeros when beta == 0)
  } else {
    const sgemm::LoadWidths w =
        load_widths(transA != 0, transB != 0, M, N, K, A, lda, strideA, B, ldb, strideB);
    const sgemm::TileChoice tile = sgemm::choose_mfma_tile(M, N, K, di.cus, batch);
    err = sgemm::launch_mfma_general(tile, p, transA, transB, w, s);
    if (err == hipErrorInvalidValue) return SGEMM_ERR_TOO_LARGE;
  }
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_run_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                 const float *A, int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                 int64_t ldc, void *stream) {
  return sgemm_run_strided_batched(transA, transB, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C,
                                   ldc, 0, 1, stream);
}

int64_t sgemm_bf16x3_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxBf16x3K) return SGEMM_ERR_TOO_LARGE;
  const int64_t Kp = (K + 31) / 32 * 32;
  if ((M + N) * Kp > kMaxBf16x3Split) return SGEMM_ERR_TOO_LARGE;
  return 6 * Kp * (M + N);  // three 2-byte planes of each operand
}

}  // extern "C"

namespace sgemm_api {

// The argument checks of sgemm_run_bf16x3_ex other than those of the
// workspace; *need receives the workspace bytes the call needs (0 when it
// reads neither A, B nor the workspace).
int bf16x3_ex_check(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                    const float *A, int64_t lda, const float *B, int64_t ldb, const float *C,
                    int64_t ldc, int64_t *need) {
  *need = 0;
  if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return SGEMM_ERR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_INVALID_VALUE;
  const int64_t a_cols = transA ? M : K, b_cols = transB ? K : N;
  if (lda < (a_cols > 1 ? a_cols : 1) || ldb < (b_cols > 1 ? b_cols : 1) ||
      ldc < (N > 1 ? N : 1))
    return SGEMM_ERR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return SGEMM_ERR_TOO_LARGE;
  if (!grid_fits(M, N, 1, 64, 64, 256)) return SGEMM_ERR_TOO_LARGE;
  const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.f;
  if (reads_ab) {
    const int64_t w = sgemm_bf16x3_workspace_size(M, N, K);
    if (w < 0) return (int)w;
    *need = w;
  }
  if (M > 0 && N > 0 && !C) return SGEMM_ERR_INVALID_VALUE;
  if (reads_ab && (!A || !B)) return SGEMM_ERR_INVALID_VALUE;
  return SGEMM_OK;
}

bool ready() { return g_ready.load(std::memory_order_acquire) != 0; }

}  // namespace sgemm_api

extern "C" {

int sgemm_run_bf16x3_ex(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                        const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                        float *C, int64_t ldc, void *workspace, int64_t workspace_bytes,
                        void *stream) {
  int64_t need = 0;
  const int chk =
      sgemm_api::bf16x3_ex_check(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, &need);
  if (chk != SGEMM_OK) return chk;
  const bool reads_ab = need > 0;
  if (reads_ab && (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return SGEMM_ERR_INVALID_VALUE;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  if (M == 0 || N == 0) return SGEMM_OK;
  DeviceInfo di;
  const int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t err;
  if (!reads_ab) {
    sgemm::GemmArgs z;
    z.M = (int)M;
    z.N = (int)N;
    z.K = (int)K;
    z.A = A;
    z.lda = lda;
    z.B = B;
    z.ldb = ldb;
    z.C = C;
    z.ldc = ldc;
    z.alpha = alpha;
    z.beta = beta;
    err = sgemm::launch_scale(z, s);  // C = beta C (zeros when beta == 0)
  } else {
    const int64_t Kp = (K + 31) / 32 * 32;
    unsigned short *wa = static_cast<unsigned short *>(workspace);
    unsigned short *wb = wa + 3 * M * Kp;
    err = sgemm::launch_split(transA != 0, transB != 0, A, lda, B, ldb, (int)M, (int)N, (int)K,
                              (int)Kp, wa, wb, s);
    if (err == hipSuccess) {
      sgemm::Bf16x3Args p;
      p.M = (int)M;
      p.N = (int)N;
      p.Kp = Kp;
      p.a = wa;
      p.b = wb;
      p.plane_a = M * Kp;
      p.plane_b = N * Kp;
      p.C = C;
      p.ldc = ldc;
      p.alpha = alpha;
      p.beta = beta;
      err = sgemm::launch_bf16x3_gemm(p, di.cus, s);
      if (err == hipErrorInvalidValue) return SGEMM_ERR_TOO_LARGE;
    }
  }
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_run_bf16x3(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                     const float *B, int64_t ldb, float *C, int64_t ldc, void *workspace,
                     int64_t workspace_bytes, void *stream) {
  return sgemm_run_bf16x3_ex(0, 0, M, N, K, 1.f, A, lda, B, ldb, 0.f, C, ldc, workspace,
                             workspace_bytes, stream);
}

int sgemm_mfma_probe(int which, const float *A, const float *B, float *C, void *stream) {
  if (which < 0 || which > 2 || !A || !B || !C) return SGEMM_ERR_INVALID_VALUE;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  DeviceInfo di;
  const int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t err = which == 2 ? sgemm::launch_bf16_probe(A, B, C, s)
                                    : sgemm::launch_mfma_probe(which, A, B, C, s);
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int vector_add(int64_t n, const float *A, const float *B, float *C, void *stream) {
  if (n < 0 || (n > 0 && (!A || !B || !C))) return SGEMM_ERR_INVALID_VALUE;
  if (n > (int64_t(1) << 33)) return SGEMM_ERR_TOO_LARGE;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  if (n == 0) return SGEMM_OK;
  DeviceInfo di;
  const int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  const hipError_t err =
      sgemm::launch_vector_add(n, A, B, C, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

int sgemm_mfma_ceiling(int which, int iters, float *out, int64_t out_len, double *flops,
                       void *stream) {
  if ((which != 0 && which != 1) || iters < 1 || !out || !flops) return SGEMM_ERR_INVALID_VALUE;
  if (!g_ready.load(std::memory_order_acquire)) return SGEMM_ERR_NOT_INITIALIZED;
  DeviceInfo di;
  const int rc = current_device_info(&di);
  if (rc != SGEMM_OK) return rc;
  if (out_len < sgemm::mfma_ceiling_outputs(di.cus)) return SGEMM_ERR_INVALID_VALUE;
  const hipError_t err = sgemm::launch_mfma_ceiling(which, iters, out, di.cus, flops,
                                                    reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? SGEMM_OK : SGEMM_ERR_LAUNCH;
}

const char *sgemm_status_string(int status) {
  switch (status) {
    case SGEMM_OK: return "SGEMM_OK";
    case SGEMM_ERR_INVALID_VALUE: return "SGEMM_ERR_INVALID_VALUE";
    case SGEMM_ERR_NOT_INITIALIZED: return "SGEMM_ERR_NOT_INITIALIZED";
    case SGEMM_ERR_UNSUPPORTED_DEVICE: return "SGEMM_ERR_UNSUPPORTED_DEVICE";
    case SGEMM_ERR_HIP: return "SGEMM_ERR_HIP";
    case SGEMM_ERR_LAUNCH: return "SGEMM_ERR_LAUNCH";
    case SGEMM_ERR_TOO_LARGE: return "SGEMM_ERR_TOO_LARGE";
    default: return "unknown status";
  }
}

const char *sgemm_variant_name(int variant) {
  switch (variant) {
    case SGEMM_VARIANT_NAIVE: return "valu_naive";
    case SGEMM_VARIANT_LDS: return "valu_lds_tiled";
    case SGEMM_VARIANT_REG: return "valu_register_tiled";
    case SGEMM_VARIANT_DBUF: return "valu_double_buffered";
    case SGEMM_VARIANT_MFMA: return "mfma_auto";
    case SGEMM_VARIANT_MFMA_256: return "mfma_256x256";
    case SGEMM_VARIANT_MFMA_128: return "mfma_128x128";
    case SGEMM_VARIANT_MFMA_64: return "mfma_64x64";
    case SGEMM_VARIANT_MFMA_32: return "mfma_32x32_ksplit4";
    case SGEMM_VARIANT_MFMA_STAGED: return "mfma_register_staged";
    case SGEMM_VARIANT_MFMA_UNPADDED: return "mfma_unpadded_lds";
    case SGEMM_VARIANT_MFMA_DWORD: return "mfma_dword_loads";
    case SGEMM_VARIANT_MFMA_32X64: return "mfma_32x64_ksplit2";
    case SGEMM_VARIANT_MFMA_SERIAL: return "mfma_serial_race_triage";
    case SGEMM_VARIANT_MFMA_16: return "mfma_16x16_ksplit4";
    case SGEMM_VARIANT_MFMA_64X96: return "mfma_64x96_ksplit2";
    default: return nullptr;
  }
}

}  // extern "C"
