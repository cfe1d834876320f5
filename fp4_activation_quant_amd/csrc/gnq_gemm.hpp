// Host entry points of the consumer GEMM (gnq_gemm.hip), called by the C ABI
// after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace gnq {

hipError_t gemm_fp8(bool mx, const void *a, const void *sa, const void *b, const void *sb,
                    const float *a_scale, const float *b_scale, int64_t M, int64_t N, int64_t K,
                    void *c, hipStream_t st);
hipError_t gemm_nvfp4(const void *a, const void *sa, const float *a_gs, const void *b, const void *sb,
                      const float *b_gs, int64_t M, int64_t N, int64_t K, void *c, hipStream_t st);

}  // namespace gnq
