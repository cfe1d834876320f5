// MFMA operand types and the direct global -> LDS copy shared by the
// consumer GEMM kernels and the fused decode kernel.
#pragma once

#include <atomic>

#include "gnq_common.hpp"

namespace gnq {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Global -> LDS DMA of 16 bytes per lane (lane l writes lds + 16 l).
__device__ __forceinline__ void dma16(const uint8_t *g, uint8_t *lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Raise a kernel's dynamic-LDS limit once per device (bit d of `done`).
inline hipError_t allow_dynamic_lds(const void *kernel, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

}  // namespace gnq
