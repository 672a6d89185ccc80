/*
 * sgemm_client.c -- a plain C99 program that uses libsgemm.so through its
 * headers only (include/sgemm.h, include/sgemm_bf16x3.h,
 * include/vector_add.h) and the HIP runtime's C API for device memory and a
 * stream.  No Python, no C++.
 *
 *     sgemm_client DIR
 *
 * DIR/case.txt holds "M N K alpha beta"; DIR/A.bin (M x K), DIR/B.bin
 * (K x N) and DIR/C0.bin (M x N) hold packed row-major float32.  The program
 * writes, into DIR:
 *   C_run.bin     sgemm_run:            C = A B
 *   C_ex.bin      sgemm_run_ex:         C = alpha A B + beta C0
 *   C_exnt.bin    sgemm_run_ex with B stored transposed (the program makes
 *                 the N x K copy on the host), alpha = 1, beta = 0
 *   C_bf16x3.bin  sgemm_run_bf16x3 with a workspace it allocates
 *   V.bin         vector_add of the first min(M K, K N) floats of A and B
 * and prints one line per call.  It also checks that a bad leading dimension
 * is refused with SGEMM_ERR_INVALID_VALUE before anything is enqueued.
 * Exit status 0 when every call returned SGEMM_OK (and the refusal came);
 * 1 otherwise; 2 for a usage or file error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sgemm.h"
#include "sgemm_bf16x3.h"
#include "vector_add.h"

static int hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int status_ok(int st, const char *what) {
  printf("%s: %s\n", what, sgemm_status_string(st));
  return st == SGEMM_OK;
}

static float *read_floats(const char *dir, const char *name, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return NULL;
  float *x = (float *)malloc(n * sizeof(float) + 1);
  if (x && fread(x, sizeof(float), n, f) != n) {
    free(x);
    x = NULL;
  }
  fclose(f);
  return x;
}

static int write_floats(const char *dir, const char *name, const float *x, size_t n) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 0;
  const int ok = fwrite(x, sizeof(float), n, f) == n;
  return fclose(f) == 0 && ok;
}

/* Copy n floats to a new device buffer (NULL on failure). */
static float *to_device(const float *h, size_t n) {
  void *d = NULL;
  if (!hip_ok(hipMalloc(&d, n * sizeof(float) + 16), "hipMalloc")) return NULL;
  if (!hip_ok(hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy")) {
    (void)hipFree(d);
    return NULL;
  }
  return (float *)d;
}

int main(int argc, char **argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char *dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/case.txt", dir);
  FILE *f = fopen(path, "r");
  long long M = 0, N = 0, K = 0;
  float alpha = 0.f, beta = 0.f;
  if (!f || fscanf(f, "%lld %lld %lld %f %f", &M, &N, &K, &alpha, &beta) != 5 || M < 1 ||
      N < 1 || K < 1) {
    fprintf(stderr, "cannot read %s\n", path);
    if (f) fclose(f);
    return 2;
  }
  fclose(f);
  const size_t nA = (size_t)(M * K), nB = (size_t)(K * N), nC = (size_t)(M * N);
  float *hA = read_floats(dir, "A.bin", nA), *hB = read_floats(dir, "B.bin", nB);
  float *hC0 = read_floats(dir, "C0.bin", nC);
  float *hBt = (float *)malloc(nB * sizeof(float) + 1);
  float *hOut = (float *)malloc(nC * sizeof(float) + 1);
  if (!hA || !hB || !hC0 || !hBt || !hOut) {
    fprintf(stderr, "cannot read the inputs in %s\n", dir);
    return 2;
  }
  for (long long k = 0; k < K; ++k)
    for (long long j = 0; j < N; ++j) hBt[j * K + k] = hB[k * N + j];

  int ok = hip_ok(hipSetDevice(0), "hipSetDevice");
  hipStream_t stream = NULL;
  ok = ok && hip_ok(hipStreamCreate(&stream), "hipStreamCreate");
  ok = ok && status_ok(sgemm_create(), "sgemm_create");
  if (!ok) return 1;

  float *dA = to_device(hA, nA), *dB = to_device(hB, nB), *dBt = to_device(hBt, nB);
  float *dC = to_device(hC0, nC), *dX = to_device(hC0, nC);
  float *dV = to_device(hC0, nC);
  const int64_t ws_bytes = sgemm_bf16x3_workspace_size(M, N, K);
  void *ws = NULL;
  if (!dA || !dB || !dBt || !dC || !dX || !dV || ws_bytes < 0 ||
      !hip_ok(hipMalloc(&ws, (size_t)ws_bytes + 16), "hipMalloc workspace"))
    return 1;

  /* Refused before anything is enqueued: lda < K. */
  const int bad = sgemm_run(M, N, K, dA, K - 1, dB, N, dC, N, stream);
  printf("sgemm_run with lda = K - 1: %s\n", sgemm_status_string(bad));
  ok = ok && bad == SGEMM_ERR_INVALID_VALUE;

  /* C_run: C = A B */
  ok = ok && status_ok(sgemm_run(M, N, K, dA, K, dB, N, dC, N, stream), "sgemm_run");
  ok = ok && hip_ok(hipStreamSynchronize(stream), "sync") &&
       hip_ok(hipMemcpy(hOut, dC, nC * sizeof(float), hipMemcpyDeviceToHost), "copy") &&
       write_floats(dir, "C_run.bin", hOut, nC);

  /* C_ex: C = alpha A B + beta C0 (dX holds C0) */
  ok = ok && status_ok(sgemm_run_ex(0, 0, M, N, K, alpha, dA, K, dB, N, beta, dX, N, stream),
                       "sgemm_run_ex");
  ok = ok && hip_ok(hipStreamSynchronize(stream), "sync") &&
       hip_ok(hipMemcpy(hOut, dX, nC * sizeof(float), hipMemcpyDeviceToHost), "copy") &&
       write_floats(dir, "C_ex.bin", hOut, nC);

  /* C_exnt: A (B^T)^T with B stored N x K */
  ok = ok && status_ok(sgemm_run_ex(0, 1, M, N, K, 1.f, dA, K, dBt, K, 0.f, dC, N, stream),
                       "sgemm_run_ex NT");
  ok = ok && hip_ok(hipStreamSynchronize(stream), "sync") &&
       hip_ok(hipMemcpy(hOut, dC, nC * sizeof(float), hipMemcpyDeviceToHost), "copy") &&
       write_floats(dir, "C_exnt.bin", hOut, nC);

  /* C_bf16x3 */
  ok = ok && status_ok(sgemm_run_bf16x3(M, N, K, dA, K, dB, N, dC, N, ws, ws_bytes, stream),
                       "sgemm_run_bf16x3");
  ok = ok && hip_ok(hipStreamSynchronize(stream), "sync") &&
       hip_ok(hipMemcpy(hOut, dC, nC * sizeof(float), hipMemcpyDeviceToHost), "copy") &&
       write_floats(dir, "C_bf16x3.bin", hOut, nC);

  /* V = A + B over the shorter of the two, written into dV (M x N floats) */
  size_t nv = nA < nB ? nA : nB;
  if (nv > nC) nv = nC;
  ok = ok && status_ok(vector_add((int64_t)nv, dA, dB, dV, stream), "vector_add");
  ok = ok && hip_ok(hipStreamSynchronize(stream), "sync") &&
       hip_ok(hipMemcpy(hOut, dV, nv * sizeof(float), hipMemcpyDeviceToHost), "copy") &&
       write_floats(dir, "V.bin", hOut, nv);

  ok = status_ok(sgemm_destroy(), "sgemm_destroy") && ok;
  (void)hipFree(ws);
  (void)hipFree(dA);
  (void)hipFree(dB);
  (void)hipFree(dBt);
  (void)hipFree(dC);
  (void)hipFree(dX);
  (void)hipFree(dV);
  (void)hipStreamDestroy(stream);
  free(hA);
  free(hB);
  free(hC0);
  free(hBt);
  free(hOut);
  printf("%s\n", ok ? "client ok" : "client FAILED");
  return ok ? 0 : 1;
}
