// Fused add + RMSNorm kernels for bf16 activations, mxfp8 output (one
// translation unit per dtype and mode so the library builds in parallel).
#include "gnq_fused.hpp"

namespace gnq {
hipError_t fused_bf16_mxfp8(const FusedArgs &a) { return dispatch_fused<Bf16, kModeMxfp8>(a); }
}  // namespace gnq
