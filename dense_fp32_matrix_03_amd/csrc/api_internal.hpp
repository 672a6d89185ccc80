// api_internal.hpp -- checks shared between the C entry points of libsgemm
// (C++ linkage, internal to the library).
#pragma once

#include <stdint.h>

namespace sgemm_api {

// The argument checks of sgemm_run_bf16x3_ex other than those of the
// workspace, in its order; *need receives the workspace bytes the call needs
// (0 when it reads neither A, B nor the workspace).  Returns SGEMM_OK or the
// status sgemm_run_bf16x3_ex would return.
int bf16x3_ex_check(int transA, int transB, int64_t M, int64_t N, int64_t K, float alpha,
                    const float *A, int64_t lda, const float *B, int64_t ldb, const float *C,
                    int64_t ldc, int64_t *need);

// Whether sgemm_create has been called (and not undone by sgemm_destroy).
bool ready();

}  // namespace sgemm_api
