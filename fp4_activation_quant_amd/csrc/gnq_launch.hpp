// Kernel launch that returns the launch's own status.
//
// hipLaunchKernel reports a bad launch in its return value, so the library
// needs no hipGetLastError after a launch: that would also report (and
// clear) an unrelated error an earlier call on the same thread had left.
#pragma once

#include <hip/hip_runtime.h>

namespace gnq {

template <class T>
struct same_type {
  using type = T;
};

// Launch `kernel` on `st` with `args` converted to the kernel's parameter
// types (the parameter types come from the kernel alone).
template <class... P>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                         typename same_type<P>::type... args) {
  void *argv[] = {(void *)&args..., nullptr};
  return hipLaunchKernel((const void *)kernel, grid, block, argv, lds, st);
}

}  // namespace gnq
