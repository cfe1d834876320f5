// Standalone FP8 / NVFP4 / MXFP8 quant entry points (both activation dtypes).
#include "gnq_quant.hpp"

namespace gnq {
hipError_t quant_bf16_fp8(const QuantArgs &a) { return run_quant<Bf16, kModeFp8>(a); }
hipError_t quant_bf16_nvfp4(const QuantArgs &a) { return run_quant<Bf16, kModeNvfp4>(a); }
hipError_t quant_fp16_fp8(const QuantArgs &a) { return run_quant<Fp16, kModeFp8>(a); }
hipError_t quant_fp16_nvfp4(const QuantArgs &a) { return run_quant<Fp16, kModeNvfp4>(a); }
hipError_t quant_bf16_mxfp8(const QuantArgs &a) { return run_quant<Bf16, kModeMxfp8>(a); }
hipError_t quant_fp16_mxfp8(const QuantArgs &a) { return run_quant<Fp16, kModeMxfp8>(a); }
}  // namespace gnq
