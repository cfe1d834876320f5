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
#include "gnq_decode.hpp"
#include "gnq_gemm.hpp"
#include "gnq_traffic.hpp"
#include "gnq_validate.hpp"

namespace gnq {
namespace {

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
    case 4: out[i] = (uint8_t)e4m3_one(div_by_scale(Bf16::lo(bits & 0xffffu), quant_scale(param, true))); break;
    case 5: out[i] = (uint8_t)e4m3_one(div_by_scale(Fp16::lo(bits & 0xffffu), quant_scale(param, true))); break;
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
    case 10:
    case 11: {
      // static FP8 quant of the 8-element chunk i / 8 by the vector routine
      // (n % 8 == 0): y = low 16 bits of patterns i & ~7 .. (i & ~7) + 7
      if (i % 8) break;
      uint32_t yb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) yb[k] = (in[i + 2 * k] & 0xffffu) | (in[i + 2 * k + 1] << 16);
      const u32x2 c = kind == 10 ? fp8_codes<Bf16>(yb, quant_scale(param, true))
                                 : fp8_codes<Fp16>(yb, quant_scale(param, true));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        out[i + k] = (uint8_t)(c[0] >> (8 * k));
        out[i + 4 + k] = (uint8_t)(c[1] >> (8 * k));
      }
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
  const nq_status v = check_op(x, residual, weight, scale, M, H, dtype, norm, mode, write_y, q, block_scale, y);
  if (v != NQ_OK || M == 0) return v;
  const bool nv = mode == NQ_MODE_NVFP4, none = mode == NQ_MODE_NONE, mx = mode == NQ_MODE_MXFP8;
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
              (hipStream_t)stream,
              nullptr};
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
  const nq_status v = check_quant(y, scale, M, H, dtype, mode, q, block_scale);
  if (v != NQ_OK || M == 0) return v;
  const bool nv = mode == NQ_MODE_NVFP4, mx = mode == NQ_MODE_MXFP8;
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
  const nq_status v = check_gemm_fp8(mx, a, sa, a_scale, b, sb, b_scale, M, N, K, out);
  if (v != NQ_OK || M == 0 || N == 0) return v;
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
  const nq_status v = check_gemm_nvfp4(a, a_scales, a_gs, b, b_scales, b_gs, M, N, K, out);
  if (v != NQ_OK || M == 0 || N == 0) return v;
  return status_of(gemm_nvfp4(a, a_scales, a_gs, b, b_scales, b_gs, M, N, K, out, (hipStream_t)stream));
}

nq_status nq_gemma_add_rms_norm_quant_gemm_fp8(const void *x, const void *residual, void *residual_out,
                                               const void *weight, float eps, const float *scale, int64_t M,
                                               int64_t H, int dtype, int write_y, void *q, void *y, const void *b,
                                               const float *b_scale, int64_t N, void *out, void *stream) {
  const nq_status v = check_fused_decode(x, residual, residual_out, weight, scale, M, H, dtype, write_y, q, y, b,
                                         b_scale, N, out);
  if (v != NQ_OK || M == 0) return v;
  FusedDecodeArgs a{x, residual, residual_out, weight, scale, eps, M, H, q, write_y ? y : nullptr,
                    b, b_scale, N, out, (hipStream_t)stream};
  return status_of(fused_decode(a, dtype == NQ_BF16));
}

nq_status nq_traffic_probe(const void *const *src, const int64_t *src_row_bytes, int nsrc,
                           void *const *dst, const int64_t *dst_row_bytes, int ndst, int64_t rows,
                           int threads, int grid, int flags, void *stream) {
  const nq_status v = check_traffic(src, src_row_bytes, nsrc, dst, dst_row_bytes, ndst, rows, threads, grid, flags);
  if (v != NQ_OK || rows == 0) return v;
  TrafficStreams t{};
  t.ndst = ndst;
  for (int i = 0; i < nsrc; ++i) {
    t.src[i] = src[i];
    t.src_chunks[i] = (unsigned)(src_row_bytes[i] / 16);
  }
  for (int i = 0; i < ndst; ++i) {
    t.dst[i] = dst[i];
    t.dst_chunks[i] = (unsigned)(dst_row_bytes[i] / 16);
  }
  return status_of(traffic_probe(t, nsrc, rows, threads, grid, (flags & NQ_PROBE_PREFETCH) != 0,
                                 (flags & NQ_PROBE_TILED_SCALES) != 0, (hipStream_t)stream));
}

nq_status nq_convert_probe(int kind, const void *in, int64_t n, float param, void *out,
                           void *stream) {
  const nq_status v = check_convert_probe(kind, in, n, param, out);
  if (v != NQ_OK || n == 0) return v;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  return status_of(launch(convert_probe, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                          kind, (const uint32_t *)in, n, param, (uint8_t *)out));
}

}  // extern "C"
