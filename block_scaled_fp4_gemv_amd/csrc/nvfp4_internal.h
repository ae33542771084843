// Library-internal declarations shared by the HIP sources of libnvfp4gemv.so
// (not exported from the shared library).
#ifndef NVFP4_INTERNAL_H
#define NVFP4_INTERNAL_H

// Records the hipError_t that nvfp4_last_hip_error reports for this thread.
__attribute__((visibility("hidden"))) void nvfp4_record_hip_error(int error);

#include <cstdint>

#include "nvfp4_gemv.h"

// The GEMV kernel with two right-hand vectors (dense B [L][2][K/2], SFB of
// two rows, C [L][2][M]); NVFP4_ERR_INVALID_SHAPE, nothing launched, where a
// K-split would be needed. Used by nvfp4_gemm_small_n for N = 2.
__attribute__((visibility("hidden"))) nvfp4_status_t nvfp4_gemv_two_vectors(
    const void *a, const void *b, const void *sfa, const void *sfb, void *c, int64_t M, int64_t K, int64_t L,
    int sf_layout, float alpha, void *stream);

#endif
