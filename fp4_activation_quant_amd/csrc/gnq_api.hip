// C ABI of the library (include/gemma_norm_quant.h): argument validation,
// the M == 0 early return, dispatch to the per-(dtype, mode) kernels, and
// the conversion probe.  The operation is `gemma_add_rms_norm_quant` on the
// `fused_norm_quant` page; its assertions (2-D contiguous bf16/fp16 x,
// residual of the same shape or None, weight of shape (H,), one fp32 scale,
// H % 64 == 0 for NVFP4) become status codes here, and nothing is launched
// or written when one fails.  The MXFP8 mode is the variant
// `allreduce_gemma_rms_norm_mxfp8` of the `fused_allreduce_gemma_rms_norm`
// page without its all-reduce; it needs H % 32 == 0.

#include <stdint.h>

#include "gemma_norm_quant.h"
#include "gnq_common.hpp"
#include "gnq_gemm.hpp"

namespace gnq {
namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x0 = (uintptr_t)a, x1 = x0 + na, y0 = (uintptr_t)b, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

bool valid_dtype(int dtype) { return dtype == NQ_BF16 || dtype == NQ_FP16; }

size_t block_scale_bytes(int64_t M, int64_t H) {
  if (M <= 0 || H < kBlock) return 0;
  const int64_t rows = (M + 127) / 128 * 128;
  const int64_t cols = ((H / kBlock) + 3) / 4 * 4;
  return (size_t)rows * (size_t)cols;
}

nq_status status_of(hipError_t e) { return e == hipSuccess ? NQ_OK : NQ_EHIP; }

// Probe: the kernels' own device routines on arbitrary 32-bit patterns.
__global__ void convert_probe(int kind, const uint32_t *__restrict__ in, int64_t n, float param,
                              uint8_t *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t bits = in[i];
  const float f = __uint_as_float(bits);
  switch (kind) {
    case 0: out[i] = (uint8_t)e4m3_one(f); break;
    case 1: {
      float v[8] = {f, 0, 0, 0, 0, 0, 0, 0};
      out[i] = (uint8_t)(e2m1x8(v) & 0xfu);
      break;
    }
    case 2: reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)(Bf16::pack(f, 0.0f) & 0xffffu); break;
    case 3: reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)(Fp16::pack(f, 0.0f) & 0xffffu); break;
    case 4: out[i] = (uint8_t)e4m3_one(div_by_scale(Bf16::lo(bits & 0xffffu), param, 1.0f / param)); break;
    case 5: out[i] = (uint8_t)e4m3_one(div_by_scale(Fp16::lo(bits & 0xffffu), param, 1.0f / param)); break;
    case 6: out[i] = (uint8_t)nvfp4_scale_code(f, param); break;
    case 7: out[i] = (uint8_t)mx_scale_code(fabsf(f)); break;
    case 8: out[i] = (uint8_t)e4m3_one(f * mx_elem_scale((uint32_t)param)); break;
    case 9: {
      // NVFP4 element step: bf16 y in bits 0..15, the block's E4M3 scale
      // code in bits 16..23, global scale `param`.
      const float o = nvfp4_elem_scale((bits >> 16) & 0xffu, param);
      float v[8] = {Bf16::lo(bits & 0xffffu) * o, 0, 0, 0, 0, 0, 0, 0};
      out[i] = (uint8_t)(e2m1x8(v) & 0xfu);
      break;
    }
    default: break;
  }
}

}  // namespace
}  // namespace gnq

using namespace gnq;

extern "C" {

int nq_abi_version(void) { return NQ_ABI_VERSION; }

const char *nq_status_string(int status) {
  switch (status) {
    case NQ_OK: return "ok";
    case NQ_EINVAL: return "invalid argument";
    case NQ_EUNSUPPORTED: return "unsupported shape or mode";
    case NQ_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t nq_block_scale_bytes(int64_t M, int64_t H) { return block_scale_bytes(M, H); }

nq_status nq_add_rms_norm_quant(const void *x, void *residual, const void *weight, float eps,
                                const float *scale, int64_t M, int64_t H, int dtype, int norm,
                                int mode, int write_y, void *q, void *block_scale, void *y,
                                void *stream) {
  if (!valid_dtype(dtype)) return NQ_EINVAL;
  if (norm != NQ_NORM_GEMMA && norm != NQ_NORM_PLAIN) return NQ_EINVAL;
  if (mode != NQ_MODE_FP8_STATIC && mode != NQ_MODE_NVFP4 && mode != NQ_MODE_NONE &&
      mode != NQ_MODE_MXFP8)
    return NQ_EINVAL;
  // H <= 2^30 and M * H <= 2^60: every byte count below fits 64 bits
  if (M < 0 || H <= 0 || H > ((int64_t)1 << 30) || M > ((int64_t)1 << 60) / H) return NQ_EINVAL;
  const bool nv = mode == NQ_MODE_NVFP4, none = mode == NQ_MODE_NONE, mx = mode == NQ_MODE_MXFP8;
  if (!x || !weight) return NQ_EINVAL;
  if (!none && !q) return NQ_EINVAL;
  if ((mode == NQ_MODE_FP8_STATIC || nv) && !scale) return NQ_EINVAL;
  if ((nv || mx) && !block_scale) return NQ_EINVAL;
  if ((write_y || none) && !y) return NQ_EINVAL;
  if (none && !write_y) return NQ_EINVAL;
  if (nv && H % 64 != 0) return NQ_EUNSUPPORTED;
  if (mx && H % kMxBlock != 0) return NQ_EUNSUPPORTED;
  // 16-bit elements need 2-byte alignment, the fp32 scale 4-byte.
  if (((uintptr_t)x | (uintptr_t)residual | (uintptr_t)weight | (uintptr_t)((write_y || none) ? y : nullptr)) % 2 != 0)
    return NQ_EINVAL;
  if ((mode == NQ_MODE_FP8_STATIC || nv) && (uintptr_t)scale % 4 != 0) return NQ_EINVAL;
  const size_t act = (size_t)M * (size_t)H * 2;
  const size_t qbytes = none ? 0 : nv ? (size_t)M * (size_t)(H / 2) : (size_t)M * (size_t)H;
  const size_t bsbytes = nv ? block_scale_bytes(M, H) : mx ? (size_t)M * (size_t)(H / kMxBlock) : 0;
  const void *yy = write_y ? y : nullptr;
  const void *qq = none ? nullptr : q;
  const void *bb = (nv || mx) ? block_scale : nullptr;
  if (residual == x) return NQ_EINVAL;
  // Written buffers may overlap nothing; read-only inputs (x, weight, the
  // scale) may overlap each other.
  const void *ss = (mode == NQ_MODE_FP8_STATIC || nv) ? (const void *)scale : nullptr;
  const void *wr[4] = {residual, qq, yy, bb};
  const size_t wlen[4] = {act, qbytes, act, bsbytes};
  const void *rd[3] = {x, weight, ss};
  const size_t rlen[3] = {act, (size_t)H * 2, 4};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(wr[i], wlen[i], wr[j], wlen[j])) return NQ_EINVAL;
    for (int k = 0; k < 3; ++k)
      if (overlaps(wr[i], wlen[i], rd[k], rlen[k])) return NQ_EINVAL;
  }
  if (M == 0) return NQ_OK;

  FusedArgs a{x,
              residual,
              weight,
              (nv || mode == NQ_MODE_FP8_STATIC) ? scale : nullptr,
              eps,
              M,
              H,
              none ? nullptr : q,
              (nv || mx) ? block_scale : nullptr,
              (write_y || none) ? y : nullptr,
              norm == NQ_NORM_GEMMA,
              (hipStream_t)stream};
  const bool bf = dtype == NQ_BF16;
  hipError_t e;
  switch (mode) {
    case NQ_MODE_NVFP4: e = bf ? fused_bf16_nvfp4(a) : fused_fp16_nvfp4(a); break;
    case NQ_MODE_MXFP8: e = bf ? fused_bf16_mxfp8(a) : fused_fp16_mxfp8(a); break;
    case NQ_MODE_NONE: e = bf ? fused_bf16_none(a) : fused_fp16_none(a); break;
    default: e = bf ? fused_bf16_fp8(a) : fused_fp16_fp8(a); break;
  }
  return status_of(e);
}

nq_status nq_gemma_add_rms_norm_quant(const void *x, void *residual, const void *weight, float eps,
                                      const float *scale, int64_t M, int64_t H, int dtype,
                                      int mode, int write_y, void *q, void *block_scale, void *y,
                                      void *stream) {
  if (mode != NQ_MODE_FP8_STATIC && mode != NQ_MODE_NVFP4) return NQ_EINVAL;
  return nq_add_rms_norm_quant(x, residual, weight, eps, scale, M, H, dtype, NQ_NORM_GEMMA, mode,
                               write_y, q, block_scale, y, stream);
}

static nq_status quant_common(const void *y, const float *scale, int64_t M, int64_t H, int dtype,
                              int mode, void *q, void *block_scale, void *stream) {
  const bool nv = mode == NQ_MODE_NVFP4, mx = mode == NQ_MODE_MXFP8;
  if (!valid_dtype(dtype)) return NQ_EINVAL;
  // H <= 2^30 and M * H <= 2^60: every byte count below fits 64 bits
  if (M < 0 || H <= 0 || H > ((int64_t)1 << 30) || M > ((int64_t)1 << 60) / H) return NQ_EINVAL;
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
  if (M == 0) return NQ_OK;
  QuantArgs a{y, mx ? nullptr : scale, M, H, q, (nv || mx) ? block_scale : nullptr,
              (hipStream_t)stream};
  const bool bf = dtype == NQ_BF16;
  hipError_t e;
  if (nv)
    e = bf ? quant_bf16_nvfp4(a) : quant_fp16_nvfp4(a);
  else if (mx)
    e = bf ? quant_bf16_mxfp8(a) : quant_fp16_mxfp8(a);
  else
    e = bf ? quant_bf16_fp8(a) : quant_fp16_fp8(a);
  return status_of(e);
}

nq_status nq_quant_fp8_static(const void *y, const float *scale, int64_t M, int64_t H, int dtype,
                              void *q, void *stream) {
  return quant_common(y, scale, M, H, dtype, NQ_MODE_FP8_STATIC, q, nullptr, stream);
}

nq_status nq_quant_nvfp4(const void *y, const float *global_scale, int64_t M, int64_t H, int dtype,
                         void *q, void *block_scale, void *stream) {
  return quant_common(y, global_scale, M, H, dtype, NQ_MODE_NVFP4, q, block_scale, stream);
}

nq_status nq_quant_mxfp8(const void *y, int64_t M, int64_t H, int dtype, void *q, void *scales,
                         void *stream) {
  return quant_common(y, nullptr, M, H, dtype, NQ_MODE_MXFP8, q, scales, stream);
}

static nq_status gemm_common(bool mx, const void *a, const void *sa, const float *a_scale,
                             const void *b, const void *sb, const float *b_scale, int64_t M,
                             int64_t N, int64_t K, void *out, void *stream) {
  if (M < 0 || N < 0 || K <= 0 || M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30) ||
      K > ((int64_t)1 << 24))
    return NQ_EINVAL;
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
  if (overlaps(out, obytes, a, abytes) || overlaps(out, obytes, b, bbytes) ||
      overlaps(out, obytes, sap, sab) || overlaps(out, obytes, sbp, sbb))
    return NQ_EINVAL;
  if (M == 0 || N == 0) return NQ_OK;
  return status_of(gemm_fp8(mx, a, mx ? sa : nullptr, b, mx ? sb : nullptr, mx ? nullptr : a_scale,
                            mx ? nullptr : b_scale, M, N, K, out, (hipStream_t)stream));
}

nq_status nq_gemm_mxfp8(const void *a, const void *a_scales, const void *b, const void *b_scales,
                        int64_t M, int64_t N, int64_t K, void *out, void *stream) {
  return gemm_common(true, a, a_scales, nullptr, b, b_scales, nullptr, M, N, K, out, stream);
}

nq_status nq_gemm_fp8_static(const void *a, const float *a_scale, const void *b,
                             const float *b_scale, int64_t M, int64_t N, int64_t K, void *out,
                             void *stream) {
  return gemm_common(false, a, nullptr, a_scale, b, nullptr, b_scale, M, N, K, out, stream);
}

nq_status nq_gemm_nvfp4(const void *a, const void *a_scales, const float *a_gs, const void *b,
                        const void *b_scales, const float *b_gs, int64_t M, int64_t N, int64_t K, void *out,
                        void *stream) {
  if (M < 0 || N < 0 || K <= 0 || M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30) ||
      K > ((int64_t)1 << 24))
    return NQ_EINVAL;
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
  if (M == 0 || N == 0) return NQ_OK;
  return status_of(gemm_nvfp4(a, a_scales, a_gs, b, b_scales, b_gs, M, N, K, out, (hipStream_t)stream));
}

nq_status nq_convert_probe(int kind, const void *in, int64_t n, float param, void *out,
                           void *stream) {
  if (kind < 0 || kind > 9 || n < 0 || n >= ((int64_t)1 << 31) || (n > 0 && (!out || !in)))
    return NQ_EINVAL;
  // kind 8 takes an E8M0 code the kernels can produce (0..247) as param.
  if (kind == 8 && !(param >= 0.0f && param <= 247.0f && param == (float)(int)param))
    return NQ_EINVAL;
  if (n == 0) return NQ_OK;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  return status_of(launch(convert_probe, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                          kind, (const uint32_t *)in, n, param, (uint8_t *)out));
}

}  // extern "C"
