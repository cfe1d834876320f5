// Sizes shared by the kernels and the host-side argument checks (no HIP
// types, so the checks also build as plain C++).
#pragma once

namespace gnq {

constexpr int kVec = 8;           // elements per thread chunk (16 bytes)
constexpr int kBlock = 16;        // elements per NVFP4 block scale
constexpr int kMxBlock = 32;      // elements per MXFP8 (E8M0) block scale
constexpr int kWave = 64;
constexpr int kMaxThreads = 1024;

}  // namespace gnq
