// Host entry of the fused decode step (gnq_decode.hip), called by the C ABI
// after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gnq {

constexpr int kFusedDecodeMaxRows = 8;
// Up to this many rows the step is one launch; above, the op and the decode
// GEMM as two launches (every workgroup of the one-launch kernel normalises
// all rows itself, which from 4 rows on costs more than the second launch).
constexpr int kFusedDecodeOneLaunchRows = 3;

struct FusedDecodeArgs {
  const void *x;
  const void *res;       // nullptr: no residual
  void *res_out;         // the updated residual (with res)
  const void *w;
  const float *scale;    // the op's static FP8 scale (also the GEMM's activation scale)
  float eps;
  int64_t M;
  int64_t H;             // = the GEMM's K
  void *q;
  void *y;               // nullptr: y not written
  const void *b;         // (N, H) FP8 weight codes
  const float *b_scale;
  int64_t N;
  void *out;             // (M, N) bf16
  hipStream_t st;
};

// Shapes the fused kernel takes (others: the op and the GEMM as two launches).
bool fused_decode_supported(int64_t M, int64_t H);
hipError_t fused_decode(const FusedDecodeArgs &a, bool bf16);

}  // namespace gnq
