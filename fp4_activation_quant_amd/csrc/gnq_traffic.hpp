// Host entry of the traffic probe (gnq_traffic.hip), called by the C ABI
// after argument validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gnq {

// Up to two read and four write streams of (rows, chunks * 16 bytes).
struct TrafficStreams {
  const void *src[2];
  unsigned src_chunks[2];
  void *dst[4];
  unsigned dst_chunks[4];
  int ndst;
};

// tiled: the last write stream is the 128x4-tiled NVFP4 block-scale layout
// (one byte per 16 elements), written as the op writes it.
hipError_t traffic_probe(const TrafficStreams &t, int nsrc, int64_t rows, int threads, int grid, bool pf,
                         bool tiled, hipStream_t st);

}  // namespace gnq
