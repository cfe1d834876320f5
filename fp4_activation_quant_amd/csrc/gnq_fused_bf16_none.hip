// Fused add + RMSNorm kernels for bf16 activations, none output (one
// translation unit per dtype and mode so the library builds in parallel).
#include "gnq_fused.hpp"

namespace gnq {
hipError_t fused_bf16_none(const FusedArgs &a) { return dispatch_fused<Bf16, kModeNone>(a); }
}  // namespace gnq
