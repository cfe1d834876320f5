// The fused kernels: residual add + (Gemma or plain) RMSNorm + FP8 / NVFP4 /
// MXFP8 / no quant, one launch.  Included by one translation unit per (dtype, mode)
// (gnq_fused_<dtype>_<mode>.hip), which instantiates GNQ_FUSED_ENTRY.
//
// Design (memory-bound; no MFMA -- nothing here is a contraction):
//  * fused_rows: one workgroup per row, grid = M (at 32768 x 8192 a grid of
//    512 to 2048 looping workgroups took 426-461 us against ~370).  The
//    exception (PF): rows of 4096 < H < 6144 at 2048 <= M <= 16384 run on
//    1024 workgroups of two chunks per thread (512 of one chunk, for rows
//    with a residual up to H = 5120) that loop over rows and issue the next
//    row's loads before the current row's reduction: 5-15% faster at M =
//    2048 ... 8192 (H = 5120), -1 ... +6% at 16384.  A thread owns 8-element
//    chunks (16 bytes) at chunk index tid, tid + nthr, ..., so every load and
//    store instruction of a wave covers contiguous memory: 1 KB of x /
//    residual / y, 512 B of FP8 codes, 256 B of FP4 codes.  1, 2 or 4 chunks
//    per thread (chunks_per_thread: one up to H = 4096, at H = 6144, 8192 and
//    for rows with a residual up to H = 5120; else two up to 16384, four up
//    to 32768).  x and residual are streamed with non-temporal loads, all
//    outputs with non-temporal stores; weight and scale are plain (L2-cached)
//    loads.  All loads of a row are issued before the first wait.  Sum of
//    squares: fp32 FMA chain per thread, DPP butterfly inside each 16-lane
//    row plus readlane across rows, one LDS slot per wave, one barrier.
//  * An NVFP4 block (16 elements) is the chunk pair held by two adjacent
//    lanes; the block amax is combined with a DPP lane swap and the even lane
//    stores the block's scale byte at its 128x4-tiled offset.  NVFP4 rows are
//    assigned to workgroups so that each 128-row scale tile is written
//    through a single XCD (nvfp4_row_of_block; in line-group order on the
//    one-chunk looping launch).
//  * An MXFP8 block (32 elements) is the chunk quad of four adjacent lanes
//    (DPP quad permutations combine the amax); the quad's first lane stores
//    the E8M0 scale byte, row-major.
//  * fused_rows_small: H <= 512, several rows per wavefront, reduced inside
//    lane groups with DPP, no LDS and no barrier.
//  * fused_rows_scalar: shapes or pointers the vector path cannot take
//    (H % 16 != 0, H > 32768, unaligned views); same arithmetic, one thread
//    per element (FP8, none) or per scale block (NVFP4, MXFP8); each value
//    rounded to the activation dtype through round1 (no fused multiply-round).
#pragma once

#include "gnq_common.hpp"

namespace gnq {

// RES_OUT: the updated residual goes to res_out instead of back into res.
// COVER: the launch guarantees nchunk == CPT * blockDim.x (every thread's
// chunks lie inside the row), so no load, sum or store is guarded.
template <class D, int MODE, bool HAS_RES, bool WRITE_Y, bool GEMMA, int CPT, bool PF, bool RES_OUT = false,
          bool COVER = false>
__global__ void __launch_bounds__(kMaxThreads)
fused_rows(const u32x4 *__restrict__ x, u32x4 *__restrict__ res, u32x4 *__restrict__ res_out,
           const u32x4 *__restrict__ w,
           const float *__restrict__ scale_ptr, float eps, int64_t M, int nchunk,
           uint8_t *__restrict__ q, uint8_t *__restrict__ bs, u32x4 *__restrict__ y, int ktiles) {
  __shared__ float partial[2][kMaxThreads / kWave];
  __shared__ float otab[MODE == kModeNvfp4 ? kNvfp4Codes : 1];
  const unsigned tid = threadIdx.x;
  const unsigned nthr = blockDim.x;
  const unsigned nch = (unsigned)nchunk;
  const int nwaves = nthr / kWave;
  // NVFP4 rows in line-group order on the looping launch of one chunk per
  // thread (residual rows: 512 workgroups, half a 1024-row span per pass).
  constexpr bool kLines = PF && CPT == 1;
  const float inv_h = __builtin_amdgcn_rcpf((float)(nchunk * kVec));
  // The row loads: x and residual stream from HBM (non-temporal).  They are
  // unconditional (a thread past the row's end re-reads its last chunk and
  // drops it), so the compiler's wait before the next row's loads into the
  // same registers counts only those loads, not the row's stores still in
  // flight.
  u32x4 xa[CPT], ra[CPT], wa[CPT];
  auto load_row = [&](int64_t b) {
    const int64_t rw = MODE == kModeNvfp4 ? nvfp4_row_of_block<kLines>(b, M) : b;
    const size_t rb = (size_t)rw * (size_t)nchunk;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = COVER ? tid + c * nthr : min(tid + c * nthr, nch - 1);
      xa[c] = __builtin_nontemporal_load(&x[rb + ch]);
      if constexpr (HAS_RES) ra[c] = __builtin_nontemporal_load(&res[rb + ch]);
    }
  };
  int64_t blk = blockIdx.x;
  if (blk < M) load_row(blk);
  // The weight and the scale come from L2, once per workgroup; the scale's
  // reciprocal is formed while the first row's loads are in flight.
#pragma unroll
  for (int c = 0; c < CPT; ++c) wa[c] = w[COVER ? tid + c * nthr : min(tid + c * nthr, nch - 1)];
  const QuantScale qs = quant_scale(mode_reads_scale(MODE) ? *scale_ptr : 1.0f, MODE == kModeFp8);
  // NVFP4: the multiplier table, read after the first row's barrier.
  if constexpr (MODE == kModeNvfp4) nvfp4_fill_table(otab, qs.s, tid, nthr);
  // The looping launch keeps the norm's per-element factor fl(1 + w) (or w)
  // in registers across its rows.
  float g[PF ? CPT : 1][PF ? kVec : 1];
  if constexpr (PF) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g[c][2 * k] = norm_factor<GEMMA>(D::lo(wa[c][k]));
        g[c][2 * k + 1] = norm_factor<GEMMA>(D::hi(wa[c][k]));
      }
  }
  int parity = 0;
  for (; blk < M; blk += gridDim.x, parity ^= 1) {
    const int64_t row = MODE == kModeNvfp4 ? nvfp4_row_of_block<kLines>(blk, M) : blk;
    const size_t rbase = (size_t)row * (size_t)nchunk;
    u32x4 *__restrict__ rr = (RES_OUT ? res_out : res) + rbase;
    u32x4 *__restrict__ yr = y + rbase;
    // h = RN(x + r), written back; sum of squares of the rounded h.
    uint32_t hb[CPT][4];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if constexpr (HAS_RES) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          hb[c][k] = D::pack(D::lo(xa[c][k]) + D::lo(ra[c][k]), D::hi(xa[c][k]) + D::hi(ra[c][k]));
        if (COVER || ch < nch) {
          const u32x4 o = {hb[c][0], hb[c][1], hb[c][2], hb[c][3]};
          __builtin_nontemporal_store(o, &rr[ch]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) hb[c][k] = xa[c][k];
      }
      // the chunk's squares, added in element order (nothing for a chunk
      // past the row's end)
      float sc = ss;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = D::lo(hb[c][k]), b = D::hi(hb[c][k]);
        sc = __builtin_fmaf(a, a, sc);
        sc = __builtin_fmaf(b, b, sc);
      }
      ss = (COVER || ch < nch) ? sc : ss;
    }
    // x and residual are dead once h is formed: with PF the next row's loads
    // go out now, behind this row's reduction and stores.
    if constexpr (PF)
      if (blk + gridDim.x < M) load_row(blk + gridDim.x);
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) partial[parity][tid / kWave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int i = 0; i < nwaves; ++i) tot += partial[parity][i];
    const float rstd = row_rstd(tot, inv_h, eps);

#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      // With PF every thread computes (a chunk past the row's end holds a
      // re-read chunk and stores nothing), so no branch separates the
      // conversions of h from their FMAs (measured: 3% faster there, 1%
      // slower without PF, where the threads past the row skip it).
      const unsigned ch = tid + c * nthr;
      const bool active = COVER || ch < nch;
      if (!PF && !active) continue;
      // y = RN(t * (1 + w)) (Gemma) or RN(t * w), t = h * rstd (as
      // fma(h, rstd, -0): the same rounding); the quant reads the rounded y.
      float y32[kVec];
      uint32_t yb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float ta = D::fma_lo(hb[c][k], rstd, qs.nz);
        const float tb = D::fma_hi(hb[c][k], rstd, qs.nz);
        if constexpr (PF) {
          y32[2 * k] = ta * g[c][2 * k];
          y32[2 * k + 1] = tb * g[c][2 * k + 1];
        } else {
          y32[2 * k] = norm_scale<GEMMA>(ta, D::lo(wa[c][k]));
          y32[2 * k + 1] = norm_scale<GEMMA>(tb, D::hi(wa[c][k]));
        }
        yb[k] = D::pack(y32[2 * k], y32[2 * k + 1]);
      }
      if constexpr (WRITE_Y)
        if (active) __builtin_nontemporal_store(u32x4{yb[0], yb[1], yb[2], yb[3]}, &yr[ch]);
      if constexpr (MODE != kModeNone)
        quant_store_chunk<D, MODE, MODE == kModeNvfp4>(yb, MODE == kModeFp8 ? 0.0f : rounded_amax<D>(y32), qs, q,
                                                       bs, row, ch, nchunk, ktiles, otab, active);
    }
    if constexpr (!PF)
      if (blk + gridDim.x < M) load_row(blk + gridDim.x);
  }
}

// Several rows per wavefront for H <= 512.  A row takes LPR lanes (the power
// of two >= H/8, one 8-element chunk per lane), a wave holds 64/LPR rows and
// a 256-thread workgroup 4 times as many.
constexpr int kSmallThreads = 256;

template <class D, int MODE, bool HAS_RES, bool WRITE_Y, bool GEMMA, int LPR>
__global__ void __launch_bounds__(kSmallThreads)
fused_rows_small(const u32x4 *__restrict__ x, u32x4 *__restrict__ res, const u32x4 *__restrict__ w,
                 const float *__restrict__ scale_ptr, float eps, int64_t M, int nchunk,
                 uint8_t *__restrict__ q, uint8_t *__restrict__ bs, u32x4 *__restrict__ y,
                 int ktiles) {
  constexpr int kRowsPerWg = kSmallThreads / LPR;
  const unsigned tid = threadIdx.x;
  const unsigned ch = tid % LPR;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWg + tid / LPR;
  const bool active = row < M && ch < (unsigned)nchunk;
  const size_t rbase = (size_t)(row < M ? row : 0) * (size_t)nchunk;
  u32x4 xa = {0, 0, 0, 0}, ra = {0, 0, 0, 0}, wa = {0, 0, 0, 0};
  if (active) {
    xa = __builtin_nontemporal_load(&x[rbase + ch]);
    if constexpr (HAS_RES) ra = __builtin_nontemporal_load(&res[rbase + ch]);
    wa = w[ch];
  }
  const QuantScale qs = quant_scale(mode_reads_scale(MODE) ? *scale_ptr : 1.0f, MODE == kModeFp8);
  uint32_t hb[4];
  float ss = 0.0f;
  if constexpr (HAS_RES) {
#pragma unroll
    for (int k = 0; k < 4; ++k) hb[k] = D::pack(D::lo(xa[k]) + D::lo(ra[k]), D::hi(xa[k]) + D::hi(ra[k]));
    if (active) {
      const u32x4 o = {hb[0], hb[1], hb[2], hb[3]};
      __builtin_nontemporal_store(o, &res[rbase + ch]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) hb[k] = xa[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = D::lo(hb[k]), b = D::hi(hb[k]);
    ss = __builtin_fmaf(a, a, ss);
    ss = __builtin_fmaf(b, b, ss);
  }
  ss = group_sum<LPR>(ss);
  const float rstd = row_rstd(ss, __builtin_amdgcn_rcpf((float)(nchunk * kVec)), eps);
  float y32[kVec];
  uint32_t yb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    y32[2 * k] = norm_scale<GEMMA>(__builtin_fmaf(D::lo(hb[k]), rstd, qs.nz), D::lo(wa[k]));
    y32[2 * k + 1] = norm_scale<GEMMA>(__builtin_fmaf(D::hi(hb[k]), rstd, qs.nz), D::hi(wa[k]));
    yb[k] = D::pack(y32[2 * k], y32[2 * k + 1]);
  }
  if constexpr (WRITE_Y) {
    if (active) {
      const u32x4 o = {yb[0], yb[1], yb[2], yb[3]};
      __builtin_nontemporal_store(o, &y[rbase + ch]);
    }
  }
  // NVFP4 has H % 64 == 0 and MXFP8 H % 32 == 0, so the lanes of a row group
  // into whole blocks (LPR >= 4 for MXFP8) and an inactive lane shares a
  // block only with inactive lanes.
  if constexpr (MODE != kModeNone)
    if (active)
      quant_store_chunk<D, MODE>(yb, MODE == kModeFp8 ? 0.0f : rounded_amax<D>(y32), qs, q, bs, row, ch, nchunk,
                                 ktiles);
}

// Any H and any alignment: element loads, same arithmetic.
template <class D, int MODE, bool HAS_RES, bool WRITE_Y, bool GEMMA>
__global__ void __launch_bounds__(256)
fused_rows_scalar(const uint16_t *__restrict__ x, uint16_t *__restrict__ res,
                  const uint16_t *__restrict__ w, const float *__restrict__ scale_ptr, float eps,
                  int64_t M, int H, uint8_t *__restrict__ q, uint8_t *__restrict__ bs,
                  uint16_t *__restrict__ y, int ktiles) {
  __shared__ float partial[2][256 / kWave];
  const int tid = threadIdx.x;
  const int nwaves = blockDim.x / kWave;
  const QuantScale qs = quant_scale(mode_reads_scale(MODE) ? *scale_ptr : 1.0f, MODE == kModeFp8);
  const float s = qs.s;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x, parity ^= 1) {
    const size_t rb = (size_t)row * (size_t)H;
    float ss = 0.0f;
    for (int j = tid; j < H; j += blockDim.x) {
      uint32_t h = x[rb + j];
      if constexpr (HAS_RES) {
        h = D::round1(D::lo(h) + D::lo(res[rb + j]));
        res[rb + j] = (uint16_t)h;
      }
      const float hf = D::lo(h);
      ss = __builtin_fmaf(hf, hf, ss);
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) partial[parity][tid / kWave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int i = 0; i < nwaves; ++i) tot += partial[parity][i];
    const float rstd = row_rstd(tot, __builtin_amdgcn_rcpf((float)H), eps);
    // After the barrier every thread may read h written by the others.
    const uint16_t *hsrc = HAS_RES ? res : x;
    if constexpr (MODE == kModeNvfp4) {
      const int nb = H / kBlock;
      for (int b = tid; b < nb; b += blockDim.x) {
        float yv[kBlock];
        for (int k = 0; k < kBlock; ++k) {
          const int j = b * kBlock + k;
          const uint32_t yq =
              D::round1(norm_scale<GEMMA>(D::lo(hsrc[rb + j]) * rstd, D::lo(w[j])));
          if constexpr (WRITE_Y) y[rb + j] = (uint16_t)yq;
          yv[k] = D::lo(yq);
        }
        float amax = 0.0f;
        for (int k = 0; k < kBlock; ++k) amax = fmaxf(amax, fabsf(yv[k]));
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
      for (int b = tid; b < nb; b += blockDim.x) {
        float yv[kMxBlock];
        for (int k = 0; k < kMxBlock; ++k) {
          const int j = b * kMxBlock + k;
          const uint32_t yq =
              D::round1(norm_scale<GEMMA>(D::lo(hsrc[rb + j]) * rstd, D::lo(w[j])));
          if constexpr (WRITE_Y) y[rb + j] = (uint16_t)yq;
          yv[k] = D::lo(yq);
        }
        bs[(size_t)row * (size_t)nb + b] = (uint8_t)mx_block_store(yv, q + rb + (size_t)b * kMxBlock);
      }
    } else {
      for (int j = tid; j < H; j += blockDim.x) {
        const uint32_t yq =
            D::round1(norm_scale<GEMMA>(D::lo(hsrc[rb + j]) * rstd, D::lo(w[j])));
        if constexpr (WRITE_Y) y[rb + j] = (uint16_t)yq;
        if constexpr (MODE == kModeFp8) q[rb + j] = (uint8_t)e4m3_one(div_by_scale(D::lo(yq), qs));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Launch: pick the kernel and shape for (M, H, alignment).

// Chunks per thread for fused_rows: one 8-element chunk per thread up to
// H = 4096 (short per-thread chains for latency), and beyond wherever that
// gives a workgroup of whole 4-wave groups within 1024 threads (H = 6144,
// 8192: its waves spread evenly over the 4 SIMDs; measured 1-3.5% faster
// than two chunks at H = 8192, while the 10-wave workgroups of H = 5120 ran
// 3-22% slower than 5-wave ones with two chunks); otherwise two up to
// H = 16384, four up to H = 32768.  The exception: rows with a residual at
// 4096 < H <= 5120 take one chunk (10-wave workgroups, two per CU on the
// looping launch: 2.7% faster there than two chunks at 4096 x 5120, with
// or without y; without a residual, 25% slower).  Every launch form of such
// a row then uses the same chunk split, so its sum of squares is formed in
// the same order whatever M is.
inline int chunks_per_thread(int64_t H, bool res) {
  const int64_t nchunk = H / kVec;
  if (H <= 4096) return 1;
  if (res && H <= 5120) return 1;
  if (nchunk <= kMaxThreads && nchunk % (4 * kWave) == 0) return 1;
  if (nchunk <= 2 * kMaxThreads) return 2;
  return 4;
}

inline bool aligned_to(const void *p, uintptr_t n) { return p == nullptr || ((uintptr_t)p % n) == 0; }

// Whether fused_rows runs as workgroups looping over rows with the next
// row's loads issued early (PF): rows of 4096 < H < 6144 at 2048 <= M <=
// 16384, where it measured faster than one workgroup per row.  1024
// workgroups of two chunks per thread (5- or 6-wave, four per CU), 512 of
// one chunk (10-wave, two per CU; 768 and 384 measured 17% and 13% slower).
// A multiple of 8 workgroups keeps each workgroup's NVFP4 rows on its own
// XCD.
constexpr int kPrefetchGrid = 1024;
constexpr int kPrefetchGridOneChunk = 512;
inline bool prefetch_rows(int64_t M, int64_t H) {
  return H > 4096 && H < 6144 && M >= 2048 && M <= 16384;
}

// Whether fused_rows / fused_rows_small can take the call.
inline bool vector_path_ok(const FusedArgs &a, int mode) {
  return (a.H % kBlock == 0) && (a.H / kVec) <= 4 * kMaxThreads && aligned_to(a.x, 16) &&
         aligned_to(a.res, 16) && aligned_to(a.w, 16) && aligned_to(a.y, 16) &&
         aligned_to(a.q, mode == kModeNvfp4 ? 4 : 8);
}

template <class D, int MODE, bool RES, bool WY, bool GEMMA>
hipError_t run_fused(const FusedArgs &a) {
  const int ktiles = (int)(((a.H / kBlock) + 3) / 4);
  const dim3 grid((unsigned)(a.M < kMaxGrid ? a.M : kMaxGrid));
  const u32x4 *x = (const u32x4 *)a.x;
  u32x4 *res = (u32x4 *)a.res;
  const u32x4 *w = (const u32x4 *)a.w;
  u32x4 *y = (u32x4 *)a.y;
  uint8_t *q = (uint8_t *)a.q, *bs = (uint8_t *)a.bs;
  if (a.res_out != nullptr) {
    // The out-of-place residual exists for the decode step's two-launch
    // form only: FP8, Gemma, rows of one chunk per thread.
    if constexpr (MODE == kModeFp8 && RES && GEMMA) {
      if (vector_path_ok(a, MODE) && aligned_to(a.res_out, 16) && a.H > 512 && chunks_per_thread(a.H, true) == 1 &&
          a.M <= kMaxGrid) {
        const int nchunk = (int)(a.H / kVec);
        const dim3 block(((nchunk + kWave - 1) / kWave) * kWave);
        return launch(fused_rows<D, MODE, RES, WY, GEMMA, 1, false, true>, grid, block, 0, a.st, x, res,
                      (u32x4 *)a.res_out, w, a.scale, a.eps, a.M, nchunk, q, bs, y, ktiles);
      }
    }
    return hipErrorInvalidValue;
  }
  if (vector_path_ok(a, MODE)) {
    const int nchunk = (int)(a.H / kVec);
    if (a.H <= 512 && a.M <= kMaxGrid) {
#define GNQ_SMALL(L)                                                                               \
  return launch(fused_rows_small<D, MODE, RES, WY, GEMMA, L>,                                       \
                dim3((unsigned)((a.M + kSmallThreads / L - 1) / (kSmallThreads / L))),            \
                dim3(kSmallThreads), 0, a.st, x, res, w, a.scale, a.eps, a.M, nchunk, q, bs, y, ktiles)
      if (nchunk <= 2) GNQ_SMALL(2);
      if (nchunk <= 4) GNQ_SMALL(4);
      if (nchunk <= 8) GNQ_SMALL(8);
      if (nchunk <= 16) GNQ_SMALL(16);
      if (nchunk <= 32) GNQ_SMALL(32);
      GNQ_SMALL(64);
#undef GNQ_SMALL
    }
    const int cpt = chunks_per_thread(a.H, RES);
    const int per_thread = (nchunk + cpt - 1) / cpt;
    const dim3 block(((per_thread + kWave - 1) / kWave) * kWave);
#define GNQ_VEC(C, P, G)                                                                               \
  return launch(fused_rows<D, MODE, RES, WY, GEMMA, C, P>, G, block, 0, a.st, x, res, nullptr, w, a.scale, \
                a.eps, a.M, nchunk, q, bs, y, ktiles)
    if (cpt == 1 && prefetch_rows(a.M, a.H)) GNQ_VEC(1, true, dim3(kPrefetchGridOneChunk));
    if (cpt == 1) GNQ_VEC(1, false, grid);
    if constexpr (!RES) {
      // Residual-free rows whose chunks the threads cover exactly (H = 5120
      // here) drop every per-chunk guard: 4-4.5% faster at 4096 x 5120 fp16
      // (with a residual the same form measured 5% slower, so it is not
      // used there).
      if (cpt == 2 && prefetch_rows(a.M, a.H) && (int)block.x * 2 == nchunk)
        return launch(fused_rows<D, MODE, RES, WY, GEMMA, 2, true, false, true>, dim3(kPrefetchGrid), block, 0,
                      a.st, x, res, nullptr, w, a.scale, a.eps, a.M, nchunk, q, bs, y, ktiles);
    }
    if (cpt == 2 && prefetch_rows(a.M, a.H)) GNQ_VEC(2, true, dim3(kPrefetchGrid));
    if (cpt == 2) GNQ_VEC(2, false, grid);
    GNQ_VEC(4, false, grid);
#undef GNQ_VEC
  }
  return launch(fused_rows_scalar<D, MODE, RES, WY, GEMMA>, grid, dim3(256), 0, a.st,
                (const uint16_t *)a.x, (uint16_t *)a.res, (const uint16_t *)a.w, a.scale, a.eps, a.M,
                (int)a.H, q, bs, (uint16_t *)a.y, ktiles);
}

template <class D, int MODE>
hipError_t dispatch_fused(const FusedArgs &a) {
  const bool res = a.res != nullptr, wy = a.y != nullptr;
  if constexpr (MODE == kModeNone) {
    // y is the only output in this mode.
    if (a.gemma) return res ? run_fused<D, MODE, true, true, true>(a) : run_fused<D, MODE, false, true, true>(a);
    return res ? run_fused<D, MODE, true, true, false>(a) : run_fused<D, MODE, false, true, false>(a);
  } else {
    if (a.gemma) {
      if (res) return wy ? run_fused<D, MODE, true, true, true>(a) : run_fused<D, MODE, true, false, true>(a);
      return wy ? run_fused<D, MODE, false, true, true>(a) : run_fused<D, MODE, false, false, true>(a);
    }
    if (res) return wy ? run_fused<D, MODE, true, true, false>(a) : run_fused<D, MODE, true, false, false>(a);
    return wy ? run_fused<D, MODE, false, true, false>(a) : run_fused<D, MODE, false, false, false>(a);
  }
}

}  // namespace gnq
