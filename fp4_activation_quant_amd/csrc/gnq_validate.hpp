// Host-side argument checks of every C-ABI entry point (include/
// gemma_norm_quant.h).  Plain C++ with no HIP types: the C ABI calls these
// before any launch, and a CPU test builds them on their own with the
// address and undefined-behaviour sanitizers and drives them through valid,
// invalid and overflow-prone arguments.
//
// Each check returns NQ_OK when the call may proceed (the caller then
// returns early for an empty problem), else the status to return with
// nothing launched or written.  The op's rules are the `fused_norm_quant`
// page's wrapper assertions (2-D contiguous x, residual of the same shape or
// none, weight of shape (H,), one fp32 scale, H % 64 == 0 for NVFP4) plus
// the aliasing rules: a written buffer overlaps no other buffer.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gemma_norm_quant.h"
#include "gnq_consts.hpp"

namespace gnq {

// Whether [a, a + na) and [b, b + nb) share a byte (empty or null ranges
// share none).  A range running past the end of the address space cannot be
// a buffer: it counts as overlapping, so the call is rejected.
inline bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x0 = (uintptr_t)a, y0 = (uintptr_t)b;
  if (na > UINTPTR_MAX - x0 || nb > UINTPTR_MAX - y0) return true;
  const uintptr_t x1 = x0 + na, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

inline bool valid_dtype(int dtype) { return dtype == NQ_BF16 || dtype == NQ_FP16; }

// H <= 2^30 and M * H <= 2^60: every byte count below fits 64 bits.
inline bool valid_rows_cols(int64_t M, int64_t H) {
  return M >= 0 && H > 0 && H <= ((int64_t)1 << 30) && M <= ((int64_t)1 << 60) / H;
}

// round_up(M, 128) * round_up(H / 16, 4); 0 for M <= 0, H < 16, or sizes
// beyond H <= 2^30 and M * H <= 2^60 (the bound of every entry point, under
// which the product fits 64 bits).
inline size_t block_scale_bytes(int64_t M, int64_t H) {
  if (M <= 0 || H < kBlock || !valid_rows_cols(M, H)) return 0;
  const int64_t rows = (M + 127) / 128 * 128;
  const int64_t cols = ((H / kBlock) + 3) / 4 * 4;
  return (size_t)rows * (size_t)cols;
}

// nq_add_rms_norm_quant (and nq_gemma_add_rms_norm_quant).
inline nq_status check_op(const void *x, const void *residual, const void *weight, const float *scale,
                          int64_t M, int64_t H, int dtype, int norm, int mode, int write_y,
                          const void *q, const void *block_scale, const void *y) {
  if (!valid_dtype(dtype)) return NQ_EINVAL;
  if (norm != NQ_NORM_GEMMA && norm != NQ_NORM_PLAIN) return NQ_EINVAL;
  if (mode != NQ_MODE_FP8_STATIC && mode != NQ_MODE_NVFP4 && mode != NQ_MODE_NONE &&
      mode != NQ_MODE_MXFP8)
    return NQ_EINVAL;
  if (!valid_rows_cols(M, H)) return NQ_EINVAL;
  const bool nv = mode == NQ_MODE_NVFP4, none = mode == NQ_MODE_NONE, mx = mode == NQ_MODE_MXFP8;
  const bool scaled = mode == NQ_MODE_FP8_STATIC || nv;
  if (!x || !weight) return NQ_EINVAL;
  if (!none && !q) return NQ_EINVAL;
  if (scaled && !scale) return NQ_EINVAL;
  if ((nv || mx) && !block_scale) return NQ_EINVAL;
  if ((write_y || none) && !y) return NQ_EINVAL;
  if (none && !write_y) return NQ_EINVAL;
  if (nv && H % 64 != 0) return NQ_EUNSUPPORTED;
  if (mx && H % kMxBlock != 0) return NQ_EUNSUPPORTED;
  // 16-bit elements need 2-byte alignment, the fp32 scale 4-byte.
  if (((uintptr_t)x | (uintptr_t)residual | (uintptr_t)weight | (uintptr_t)((write_y || none) ? y : nullptr)) %
          2 != 0)
    return NQ_EINVAL;
  if (scaled && (uintptr_t)scale % 4 != 0) return NQ_EINVAL;
  const size_t act = (size_t)M * (size_t)H * 2;
  const size_t qbytes = none ? 0 : nv ? (size_t)M * (size_t)(H / 2) : (size_t)M * (size_t)H;
  const size_t bsbytes = nv ? block_scale_bytes(M, H) : mx ? (size_t)M * (size_t)(H / kMxBlock) : 0;
  if (residual == x) return NQ_EINVAL;
  // Written buffers may overlap nothing; read-only inputs (x, weight, the
  // scale) may overlap each other.
  const void *wr[4] = {residual, none ? nullptr : q, write_y ? y : nullptr, (nv || mx) ? block_scale : nullptr};
  const size_t wlen[4] = {act, qbytes, act, bsbytes};
  const void *rd[3] = {x, weight, scaled ? (const void *)scale : nullptr};
  const size_t rlen[3] = {act, (size_t)H * 2, 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(wr[i], wlen[i], wr[j], wlen[j])) return NQ_EINVAL;
    for (int k = 0; k < 3; ++k)
      if (overlaps(wr[i], wlen[i], rd[k], rlen[k])) return NQ_EINVAL;
  }
  return NQ_OK;
}

// nq_quant_fp8_static / nq_quant_nvfp4 / nq_quant_mxfp8.
inline nq_status check_quant(const void *y, const float *scale, int64_t M, int64_t H, int dtype, int mode,
                             const void *q, const void *block_scale) {
  const bool nv = mode == NQ_MODE_NVFP4, mx = mode == NQ_MODE_MXFP8;
  if (!valid_dtype(dtype)) return NQ_EINVAL;
  if (!valid_rows_cols(M, H)) return NQ_EINVAL;
  if (!y || !q || (!mx && !scale) || ((nv || mx) && !block_scale)) return NQ_EINVAL;
  if (nv && H % kBlock != 0) return NQ_EUNSUPPORTED;
  if (mx && H % kMxBlock != 0) return NQ_EUNSUPPORTED;
  if ((uintptr_t)y % 2 != 0 || (!mx && (uintptr_t)scale % 4 != 0)) return NQ_EINVAL;
  const size_t act = (size_t)M * (size_t)H * 2;
  const size_t qbytes = nv ? (size_t)M * (size_t)(H / 2) : (size_t)M * (size_t)H;
  const size_t bsbytes = nv ? block_scale_bytes(M, H) : mx ? (size_t)M * (size_t)(H / kMxBlock) : 0;
  const void *ss = mx ? nullptr : (const void *)scale;
  const void *bb = (nv || mx) ? block_scale : nullptr;
  if (overlaps(y, act, q, qbytes) || overlaps(y, act, bb, bsbytes) || overlaps(q, qbytes, bb, bsbytes) ||
      overlaps(ss, 4, q, qbytes) || overlaps(ss, 4, bb, bsbytes))
    return NQ_EINVAL;
  return NQ_OK;
}

inline bool valid_gemm_dims(int64_t M, int64_t N, int64_t K) {
  return M >= 0 && N >= 0 && K > 0 && M <= ((int64_t)1 << 30) && N <= ((int64_t)1 << 30) &&
         K <= ((int64_t)1 << 24);
}

// nq_gemm_mxfp8 (mx) / nq_gemm_fp8_static.
inline nq_status check_gemm_fp8(bool mx, const void *a, const void *sa, const float *a_scale, const void *b,
                                const void *sb, const float *b_scale, int64_t M, int64_t N, int64_t K,
                                const void *out) {
  if (!valid_gemm_dims(M, N, K)) return NQ_EINVAL;
  if (!a || !b || !out) return NQ_EINVAL;
  if (mx ? (!sa || !sb) : (!a_scale || !b_scale)) return NQ_EINVAL;
  if (K % kMxBlock != 0) return NQ_EUNSUPPORTED;
  if (((uintptr_t)a | (uintptr_t)b) % 16 != 0 || (uintptr_t)out % 2 != 0) return NQ_EINVAL;
  if (!mx && ((uintptr_t)a_scale | (uintptr_t)b_scale) % 4 != 0) return NQ_EINVAL;
  // one workgroup per 256 x 256 output tile: the count must fit a grid
  if (((M + 255) / 256) * ((N + 255) / 256) > (int64_t)INT32_MAX) return NQ_EINVAL;
  const size_t obytes = (size_t)M * (size_t)N * 2;
  const size_t abytes = (size_t)M * (size_t)K, bbytes = (size_t)N * (size_t)K;
  const size_t sab = mx ? (size_t)M * (size_t)(K / kMxBlock) : 4;
  const size_t sbb = mx ? (size_t)N * (size_t)(K / kMxBlock) : 4;
  const void *sap = mx ? sa : (const void *)a_scale, *sbp = mx ? sb : (const void *)b_scale;
  if (overlaps(out, obytes, a, abytes) || overlaps(out, obytes, b, bbytes) || overlaps(out, obytes, sap, sab) ||
      overlaps(out, obytes, sbp, sbb))
    return NQ_EINVAL;
  return NQ_OK;
}

// nq_gemm_nvfp4.
inline nq_status check_gemm_nvfp4(const void *a, const void *a_scales, const float *a_gs, const void *b,
                                  const void *b_scales, const float *b_gs, int64_t M, int64_t N, int64_t K,
                                  const void *out) {
  if (!valid_gemm_dims(M, N, K)) return NQ_EINVAL;
  if (!a || !b || !a_scales || !b_scales || !a_gs || !b_gs || !out) return NQ_EINVAL;
  if (K % 64 != 0) return NQ_EUNSUPPORTED;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)a_scales | (uintptr_t)b_scales) % 16 != 0 ||
      (uintptr_t)out % 2 != 0 || ((uintptr_t)a_gs | (uintptr_t)b_gs) % 4 != 0)
    return NQ_EINVAL;
  // one workgroup per 32 x 32 (or larger) output tile: the count must fit a grid
  if (((M + 31) / 32) * ((N + 31) / 32) > (int64_t)INT32_MAX) return NQ_EINVAL;
  const size_t obytes = (size_t)M * (size_t)N * 2;
  if (overlaps(out, obytes, a, (size_t)M * (size_t)(K / 2)) || overlaps(out, obytes, b, (size_t)N * (size_t)(K / 2)) ||
      overlaps(out, obytes, a_scales, block_scale_bytes(M, K)) ||
      overlaps(out, obytes, b_scales, block_scale_bytes(N, K)) || overlaps(out, obytes, a_gs, 4) ||
      overlaps(out, obytes, b_gs, 4))
    return NQ_EINVAL;
  return NQ_OK;
}

// nq_gemma_add_rms_norm_quant_gemm_fp8: the op in static FP8 mode on M <= 8
// rows with H in {1024, 2048, 4096} (NQ_EUNSUPPORTED otherwise, also for
// N == 0: the two-launch path covers those), and its consumer GEMM.  The
// updated residual goes to residual_out, which must not overlap anything
// (in particular not residual).
inline nq_status check_fused_decode(const void *x, const void *residual, const void *residual_out,
                                    const void *weight, const float *scale, int64_t M, int64_t H, int dtype,
                                    int write_y, const void *q, const void *y, const void *b,
                                    const float *b_scale, int64_t N, const void *out) {
  if (!valid_dtype(dtype)) return NQ_EINVAL;
  if (M < 0 || H <= 0 || N < 0 || N > ((int64_t)1 << 30) || H > ((int64_t)1 << 30)) return NQ_EINVAL;
  if (!x || !weight || !scale || !q || !b || !b_scale || !out) return NQ_EINVAL;
  if ((residual != nullptr) != (residual_out != nullptr)) return NQ_EINVAL;
  if (write_y && !y) return NQ_EINVAL;
  if (M == 0) return NQ_OK;
  if (M > 8 || N == 0 || !(H == 1024 || H == 2048 || H == 4096)) return NQ_EUNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)residual | (uintptr_t)residual_out | (uintptr_t)weight |
       (uintptr_t)(write_y ? y : nullptr) | (uintptr_t)b) % 16 != 0 ||
      (uintptr_t)q % 8 != 0 || (uintptr_t)out % 2 != 0 || ((uintptr_t)scale | (uintptr_t)b_scale) % 4 != 0)
    return NQ_EINVAL;
  const size_t act = (size_t)M * (size_t)H * 2;
  const void *wr[4] = {residual_out, q, write_y ? y : nullptr, out};
  const size_t wlen[4] = {act, (size_t)M * (size_t)H, act, (size_t)M * (size_t)N * 2};
  const void *rd[6] = {x, residual, weight, scale, b, b_scale};
  const size_t rlen[6] = {act, act, (size_t)H * 2, 4, (size_t)N * (size_t)H, 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(wr[i], wlen[i], wr[j], wlen[j])) return NQ_EINVAL;
    for (int k = 0; k < 6; ++k)
      if (overlaps(wr[i], wlen[i], rd[k], rlen[k])) return NQ_EINVAL;
  }
  return NQ_OK;
}

// nq_traffic_probe: 1..2 read and 0..4 write streams of 16-byte chunks, a
// read row within 4 chunks per thread; no write stream overlaps another
// stream; flags from NQ_PROBE_PREFETCH | NQ_PROBE_TILED_SCALES, the tiled
// scale stream (the last write stream) on whole 128-row tiles.
inline nq_status check_traffic(const void *const *src, const int64_t *src_row_bytes, int nsrc,
                               void *const *dst, const int64_t *dst_row_bytes, int ndst, int64_t rows,
                               int threads, int grid, int flags) {
  if (nsrc < 1 || nsrc > 2 || ndst < 0 || ndst > 4 || rows < 0 || !src || !src_row_bytes ||
      (ndst > 0 && (!dst || !dst_row_bytes)))
    return NQ_EINVAL;
  if ((flags & ~(NQ_PROBE_PREFETCH | NQ_PROBE_TILED_SCALES)) != 0) return NQ_EINVAL;
  if ((flags & NQ_PROBE_TILED_SCALES) != 0 && (ndst < 1 || rows % 128 != 0)) return NQ_EINVAL;
  if (threads < kWave || threads > kMaxThreads || threads % kWave != 0 || grid < 0) return NQ_EINVAL;
  const void *bufs[6];
  size_t lens[6];
  for (int i = 0; i < nsrc + ndst; ++i) {
    const bool is_src = i < nsrc;
    const void *p = is_src ? src[i] : dst[i - nsrc];
    const int64_t rb = is_src ? src_row_bytes[i] : dst_row_bytes[i - nsrc];
    if (!p || (uintptr_t)p % 16 != 0 || rb <= 0 || rb % 16 != 0) return NQ_EINVAL;
    if (rb / 16 > (is_src ? (int64_t)4 * threads : (int64_t)1 << 30)) return NQ_EINVAL;
    if (rows > ((int64_t)1 << 60) / rb) return NQ_EINVAL;
    bufs[i] = p;
    lens[i] = (size_t)rows * (size_t)rb;
  }
  for (int i = nsrc; i < nsrc + ndst; ++i)
    for (int j = 0; j < nsrc + ndst; ++j)
      if (j != i && overlaps(bufs[i], lens[i], bufs[j], lens[j])) return NQ_EINVAL;
  return NQ_OK;
}

// nq_convert_probe: kinds 0..9, n in [0, 2^31); kind 8 takes an E8M0 code
// the kernels can produce (an integer in 0..247) as its parameter.
inline nq_status check_convert_probe(int kind, const void *in, int64_t n, float param, const void *out) {
  if (kind < 0 || kind > 11 || n < 0 || n >= ((int64_t)1 << 31) || (n > 0 && (!out || !in))) return NQ_EINVAL;
  if (kind >= 10 && n % 8 != 0) return NQ_EINVAL;
  if (kind == 8 && !(param >= 0.0f && param <= 247.0f && param == (float)(int)param)) return NQ_EINVAL;
  return NQ_OK;
}

}  // namespace gnq
