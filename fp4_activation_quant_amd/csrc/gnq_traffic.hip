// Traffic probe: a kernel that moves the bytes of one launch of the op, with
// the op's access structure and none of its arithmetic, so the bandwidth a
// launch of that size and read / write mix can reach is measured on the same
// hardware with the same timing.  It is a measuring instrument (the
// practical ceiling the op's HBM figures are compared with), not part of
// the op.
//
// Per row: every thread issues non-temporal 16-byte loads of its chunks of
// each read stream (chunk index tid, tid + nthr, ...: a wave's load covers
// contiguous memory), folds them into one value (so no load can be dropped)
// and writes that value to its chunks of each write stream with
// non-temporal stores.  Rows go to workgroups one per row (grid = rows) or
// round-robin over a fixed grid; with PF the next row's loads are issued
// before the current row's stores, as in the op's looping launch.  With
// TILED the last write stream holds one byte per 16-element block in the
// 128x4-tiled NVFP4 block-scale layout, stored as the op stores it (plain
// byte stores at the tiled offsets, one per pair of 8-element chunks, from
// the pair's even thread), and rows take the op's NVFP4 row order (each
// 128-row tile through one XCD).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gnq_common.hpp"
#include "gnq_traffic.hpp"

namespace gnq {
namespace {

template <int NSRC, int CPT, bool PF, bool TILED>
__global__ void __launch_bounds__(kMaxThreads)
traffic_rows(TrafficStreams t, int64_t rows) {
  const unsigned tid = threadIdx.x, nthr = blockDim.x;
  u32x4 v[NSRC][CPT];
  auto row_of = [&](int64_t b) { return TILED ? nvfp4_row_of_block(b, rows) : b; };
  auto load_row = [&](int64_t b) {
    const int64_t row = row_of(b);
#pragma unroll
    for (int s = 0; s < NSRC; ++s) {
      const u32x4 *src = (const u32x4 *)t.src[s] + (size_t)row * t.src_chunks[s];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const unsigned ch = tid + c * nthr;
        v[s][c] = ch < t.src_chunks[s] ? __builtin_nontemporal_load(&src[ch]) : u32x4{0, 0, 0, 0};
      }
    }
  };
  int64_t blk = blockIdx.x;
  if (blk < rows) load_row(blk);
  for (; blk < rows; blk += gridDim.x) {
    const int64_t row = row_of(blk);
    u32x4 acc = {(uint32_t)row, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < NSRC; ++s)
#pragma unroll
      for (int c = 0; c < CPT; ++c) acc ^= v[s][c];
    if constexpr (PF)
      if (blk + gridDim.x < rows) load_row(blk + gridDim.x);
    const int nplain = TILED ? t.ndst - 1 : t.ndst;
    for (int d = 0; d < nplain; ++d) {
      u32x4 *dst = (u32x4 *)t.dst[d] + (size_t)row * t.dst_chunks[d];
      for (unsigned ch = tid; ch < t.dst_chunks[d]; ch += nthr)
        __builtin_nontemporal_store(acc ^ ch, &dst[ch]);
    }
    if constexpr (TILED) {
      // one byte per block: 16 bytes of the stream's row are 16 blocks,
      // i.e. 32 chunks of 8 elements, whose even threads store
      const unsigned nblk = t.dst_chunks[t.ndst - 1] * 16u, ktiles = nblk / 4u;
      uint8_t *bs = (uint8_t *)t.dst[t.ndst - 1] + swz128x4_row(row, (int)ktiles);
      for (unsigned ch = tid; ch < 2u * nblk; ch += nthr)
        if ((ch & 1u) == 0) bs[swz128x4_col((int)(ch >> 1))] = (uint8_t)(acc[0] ^ (ch >> 1));
    }
    if constexpr (!PF)
      if (blk + gridDim.x < rows) load_row(blk + gridDim.x);
  }
}

}  // namespace

template <bool TILED>
hipError_t traffic_probe_t(const TrafficStreams &t, int nsrc, int64_t rows, int threads, int grid, bool pf,
                           hipStream_t st) {
  unsigned most = 0;
  for (int s = 0; s < nsrc; ++s) most = t.src_chunks[s] > most ? t.src_chunks[s] : most;
  const int cpt = (int)((most + threads - 1) / threads);
  const dim3 g((unsigned)(grid > 0 ? grid : (rows < kMaxGrid ? rows : kMaxGrid))), b((unsigned)threads);
#define GNQ_TP(N, C, P) return launch(traffic_rows<N, C, P, TILED>, g, b, 0, st, t, rows)
#define GNQ_TP_CPT(N, P)          \
  if (cpt <= 1) GNQ_TP(N, 1, P);  \
  if (cpt <= 2) GNQ_TP(N, 2, P);  \
  GNQ_TP(N, 4, P)
  if (nsrc == 1) {
    if (pf) { GNQ_TP_CPT(1, true); }
    GNQ_TP_CPT(1, false);
  }
  if (pf) { GNQ_TP_CPT(2, true); }
  GNQ_TP_CPT(2, false);
#undef GNQ_TP_CPT
#undef GNQ_TP
}

hipError_t traffic_probe(const TrafficStreams &t, int nsrc, int64_t rows, int threads, int grid, bool pf,
                         bool tiled, hipStream_t st) {
  if (tiled) return traffic_probe_t<true>(t, nsrc, rows, threads, grid, pf, st);
  return traffic_probe_t<false>(t, nsrc, rows, threads, grid, pf, st);
}

}  // namespace gnq
