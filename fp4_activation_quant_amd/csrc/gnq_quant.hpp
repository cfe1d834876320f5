// Standalone quant kernels: the second kernel of the unfused chain (an
// activation already normalised and rounded to its dtype -> static FP8 codes,
// NVFP4 codes + 128x4-tiled E4M3 block scales, or MXFP8 codes + row-major
// E8M0 scales), with the same arithmetic and the same launch geometry as the
// fused kernels' quant step.
#pragma once

#include "gnq_common.hpp"

namespace gnq {

template <class D, int MODE, int CPT>
__global__ void __launch_bounds__(kMaxThreads)
quant_rows(const u32x4 *__restrict__ y, const float *__restrict__ scale_ptr, int64_t M, int nchunk,
           uint8_t *__restrict__ q, uint8_t *__restrict__ bs, int ktiles) {
  const unsigned tid = threadIdx.x;
  const unsigned nthr = blockDim.x;
  const unsigned nch = (unsigned)nchunk;
  // NVFP4: the fused kernel's multiplier table (same values as dividing).
  __shared__ float otab[MODE == kModeNvfp4 ? kNvfp4Codes : 1];
  if constexpr (MODE == kModeNvfp4) {
    nvfp4_fill_table(otab, *scale_ptr, tid, nthr);
    __syncthreads();
  }
  for (int64_t blk = blockIdx.x; blk < M; blk += gridDim.x) {
    const int64_t row = MODE == kModeNvfp4 ? nvfp4_row_of_block(blk, M) : blk;
    const u32x4 *__restrict__ yr = y + (size_t)row * (size_t)nchunk;
    u32x4 ya[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) ya[c] = __builtin_nontemporal_load(&yr[ch]);
    }
    const QuantScale qs = quant_scale(mode_reads_scale(MODE) ? *scale_ptr : 1.0f, MODE == kModeFp8);
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) {
        const uint32_t yb[4] = {ya[c][0], ya[c][1], ya[c][2], ya[c][3]};
        quant_store_chunk<D, MODE, MODE == kModeNvfp4>(yb, MODE == kModeFp8 ? 0.0f : chunk_amax<D>(yb), qs, q, bs,
                                                       row, ch, nchunk, ktiles, otab);
      }
    }
  }
}

template <class D, int MODE>
__global__ void __launch_bounds__(256)
quant_rows_scalar(const uint16_t *__restrict__ y, const float *__restrict__ scale_ptr, int64_t M,
                  int H, uint8_t *__restrict__ q, uint8_t *__restrict__ bs, int ktiles) {
  const QuantScale qs = quant_scale(mode_reads_scale(MODE) ? *scale_ptr : 1.0f, MODE == kModeFp8);
  const float s = qs.s;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    const size_t rb = (size_t)row * (size_t)H;
    if constexpr (MODE == kModeNvfp4) {
      const int nb = H / kBlock;
      for (int b = threadIdx.x; b < nb; b += blockDim.x) {
        float yv[kBlock];
        float amax = 0.0f;
        for (int k = 0; k < kBlock; ++k) {
          yv[k] = D::lo(y[rb + (size_t)b * kBlock + k]);
          amax = fmaxf(amax, fabsf(yv[k]));
        }
        const uint32_t sc = nvfp4_scale_code(amax, s);
        const float o = nvfp4_elem_scale(sc, s);
        float v[kBlock];
        for (int k = 0; k < kBlock; ++k) v[k] = yv[k] * o;
        const uint32_t p0 = e2m1x8(v), p1 = e2m1x8(v + 8);
        uint8_t *qp = q + (size_t)row * (size_t)(H / 2) + (size_t)b * 8;
        for (int k = 0; k < 4; ++k) {
          qp[k] = (uint8_t)(p0 >> (8 * k));
          qp[4 + k] = (uint8_t)(p1 >> (8 * k));
        }
        bs[swz128x4(row, b, ktiles)] = (uint8_t)sc;
      }
    } else if constexpr (MODE == kModeMxfp8) {
      const int nb = H / kMxBlock;
      for (int b = threadIdx.x; b < nb; b += blockDim.x) {
        float yv[kMxBlock];
        for (int k = 0; k < kMxBlock; ++k) yv[k] = D::lo(y[rb + (size_t)b * kMxBlock + k]);
        bs[(size_t)row * (size_t)nb + b] = (uint8_t)mx_block_store(yv, q + rb + (size_t)b * kMxBlock);
      }
    } else {
      for (int j = threadIdx.x; j < H; j += blockDim.x)
        q[rb + j] = (uint8_t)e4m3_one(div_by_scale(D::lo(y[rb + j]), qs));
    }
  }
}

template <class D, int MODE>
hipError_t run_quant(const QuantArgs &a) {
  const int ktiles = (int)(((a.H / kBlock) + 3) / 4);
  const dim3 grid((unsigned)(a.M < kMaxGrid ? a.M : kMaxGrid));
  const bool vec = (a.H % kBlock == 0) && (a.H / kVec) <= 4 * kMaxThreads &&
                   ((uintptr_t)a.y % 16) == 0 && ((uintptr_t)a.q % (MODE == kModeNvfp4 ? 4 : 8)) == 0;
  if (vec) {
    const int nchunk = (int)(a.H / kVec);
    const int cpt = nchunk <= kMaxThreads ? 1 : (nchunk <= 2 * kMaxThreads ? 2 : 4);
    const int per_thread = (nchunk + cpt - 1) / cpt;
    const dim3 block(((per_thread + kWave - 1) / kWave) * kWave);
#define GNQ_QV(C)                                                                              \
  return launch(quant_rows<D, MODE, C>, grid, block, 0, a.st, (const u32x4 *)a.y, a.scale, a.M, \
                nchunk, (uint8_t *)a.q, (uint8_t *)a.bs, ktiles)
    if (cpt == 1) GNQ_QV(1);
    if (cpt == 2) GNQ_QV(2);
    GNQ_QV(4);
#undef GNQ_QV
  }
  return launch(quant_rows_scalar<D, MODE>, grid, dim3(256), 0, a.st, (const uint16_t *)a.y, a.scale,
                a.M, (int)a.H, (uint8_t *)a.q, (uint8_t *)a.bs, ktiles);
}

}  // namespace gnq
