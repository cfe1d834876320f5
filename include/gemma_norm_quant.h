/*
 * gemma_norm_quant.h -- C ABI of the MI355X (gfx950) fused residual-add +
 * Gemma RMSNorm + activation-quant library (libgemma_norm_quant.so).
 *
 * The operation is `gemma_add_rms_norm_quant` on the `fused_norm_quant`
 * page (its argument list, return tuple and Python wrapper):
 *
 *   h        = x + residual, rounded to x's dtype and stored back into
 *              `residual` (the residual stream is updated in place); h = x
 *              when residual is NULL, and nothing is stored back then;
 *   y        = h * rsqrt(mean(h^2) + eps) * (1 + weight), fp32 arithmetic,
 *              rounded to x's dtype (Gemma's norm multiplies by one plus the
 *              weight; the codes below are taken from this rounded y, as
 *              the page's module docstring states);
 *   FP8      : q = E4M3FN(clamp(y / scale, -448, 448)), round to nearest even
 *              (static per-tensor scale; the caller keeps `scale` as the
 *              returned block scale);
 *   NVFP4    : per 16-element block of a row, a = max|y|, S = E4M3FN(min(
 *              scale * (a / 6), 448)), o = scale / S (0 if S == 0), codes
 *              E2M1(clamp(y * o, -6, 6)) round to nearest even, two per byte
 *              with the even-index element in the low nibble (the operand
 *              order of the page's `_cvt_e2m1x2` helper); S is stored in the 128x4-tiled
 *              layout (byte (m, b) at ((m/128)*(Kp/4) + b/4)*512 +
 *              (m%32)*16 + ((m%128)/32)*4 + b%4, Kp = round_up(H/16, 4));
 *              rows >= M of that buffer are never written.
 *
 * Around it the library also exports the op's variants and its unfused form:
 * the same add + RMSNorm with a plain (w instead of 1 + w) norm, with no
 * quant, or with an MXFP8 output (the `allreduce_gemma_rms_norm_mxfp8`
 * variant on the `fused_allreduce_gemma_rms_norm` page, without its
 * all-reduce), and the standalone FP8 / NVFP4 / MXFP8 quant of an
 * activation.  MXFP8 takes the OCP Microscaling scale rule (the page gives
 * only the outputs' types and shapes): per 32-element block of a row,
 * a = max|y|, e = max(floor(log2 a) - 8, -127) (-127 for a = 0), E8M0 scale
 * code e + 127, codes E4M3FN(clamp(y * 2^-e, -448, 448)) round to nearest
 * even; codes (M, H) and scales (M, H/32) both row-major.
 *
 * All pointers are caller-owned device buffers on the current HIP device.
 * The library allocates nothing, keeps no pointer past the call and launches
 * asynchronously on `stream` (a hipStream_t; NULL is the null stream).  On
 * any error nothing is launched and nothing is written.  No C++ exception
 * crosses this boundary.  NQ_EHIP is the status of this call's own HIP
 * calls (the launch's return value): an error an earlier call left on the
 * thread is neither reported nor cleared.
 *
 * Library state: none for the norm / quant entry points.  The GEMM entry
 * points raise their kernels' dynamic-LDS limit (hipFuncSetAttribute) on
 * the first call on each device and remember that in a process-wide atomic
 * bit set per kernel (devices 0..63); concurrent first calls may both set
 * the attribute, which is harmless.  Nothing else persists between calls.
 */
#ifndef GEMMA_NORM_QUANT_H
#define GEMMA_NORM_QUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NQ_ABI_VERSION 7

typedef enum {
  NQ_OK = 0,
  NQ_EINVAL = 1,        /* null required pointer, bad size, bad enum, aliasing */
  NQ_EUNSUPPORTED = 2,  /* NVFP4 with H % 64 != 0 (H % 16 != 0 for the standalone quant),
                           MXFP8 with H % 32 != 0 */
  NQ_EHIP = 3           /* a HIP runtime call or the launch failed */
} nq_status;

typedef enum { NQ_BF16 = 0, NQ_FP16 = 1 } nq_dtype;

typedef enum {
  NQ_MODE_FP8_STATIC = 0,
  NQ_MODE_NVFP4 = 1,
  NQ_MODE_NONE = 2,
  NQ_MODE_MXFP8 = 3
} nq_mode;

/* RMSNorm scaling: Gemma's (1 + weight), or plain weight. */
typedef enum { NQ_NORM_GEMMA = 0, NQ_NORM_PLAIN = 1 } nq_norm;

/*
 * nq_gemma_add_rms_norm_quant -- the op above, one launch.
 *
 *   x          (M, H) dtype, row-major contiguous, read only.
 *   residual   (M, H) dtype or NULL; updated in place to x + residual.
 *              Must not be the same buffer as x.
 *   weight     (H,) dtype; the norm scales by (1 + weight).
 *   eps        RMS-norm epsilon (> 0; eps == 0 with an all-zero row gives
 *              NaN, as the definition does).
 *   scale      DEVICE pointer to one fp32: FP8 mode, the static per-tensor
 *              scale (> 0); NVFP4 mode, the global scale (> 0) that maps a
 *              block's amax/6 into E4M3's range (448*6/amax for a tensor
 *              amax).  Non-finite values are outside the contract.
 *   M, H       rows (tokens) >= 0 and hidden size 1 .. 2^30, with
 *              M * H <= 2^60 (NQ_EINVAL otherwise).  M == 0 returns
 *              NQ_OK without launching.  NVFP4 needs H % 64 == 0 (whole
 *              4-column scale tiles, so no padded scale columns exist).
 *   dtype      nq_dtype of x, residual, weight and y.
 *   mode       nq_mode.
 *   write_y    nonzero: also write y.
 *   q          FP8: (M, H) bytes of E4M3FN codes.  NVFP4: (M, H/2) bytes of
 *              packed E2M1 codes.
 *   block_scale NVFP4: nq_block_scale_bytes(M, H) bytes, 128x4-tiled E4M3FN
 *              block scales; bytes of rows >= M are left as they were.
 *              FP8: ignored (may be NULL).
 *   y          (M, H) dtype when write_y, else ignored (may be NULL).
 *   stream     hipStream_t to launch on.
 *
 * Outputs (residual, q, block_scale, y) must not overlap each other or an
 * input (x, weight, and the fp32 scale in FP8 / NVFP4 modes); read-only
 * inputs may overlap each other (NQ_EINVAL otherwise, nothing written).
 * x, residual, weight and y must be 2-byte aligned and scale 4-byte aligned
 * (NQ_EINVAL otherwise); any H is accepted.  The fast path needs 16-byte
 * aligned pointers and H % 16 == 0, other cases take a slower correct path.
 */
nq_status nq_gemma_add_rms_norm_quant(const void *x, void *residual, const void *weight,
                                      float eps, const float *scale, int64_t M, int64_t H,
                                      int dtype, int mode, int write_y, void *q,
                                      void *block_scale, void *y, void *stream);

/*
 * nq_add_rms_norm_quant -- the same op with the norm and the output chosen:
 *
 *   norm   NQ_NORM_GEMMA: y scales by (1 + weight), as above;
 *          NQ_NORM_PLAIN: y scales by weight (plain RMSNorm, the
 *          `rms_norm_static_fp8_quant` / `fused_add_rms_norm_static_fp8_quant`
 *          semantics named on the PR conversation page).
 *   mode   NQ_MODE_FP8_STATIC / NQ_MODE_NVFP4 as above, or NQ_MODE_NONE: no
 *          quant, the op is add + RMSNorm alone (what
 *          `fused_allreduce_gemma_rms_norm` reduces to at tensor-parallel
 *          size 1, where it equals the unfused path); then write_y must be
 *          nonzero and y non-NULL, and scale, q
 *          and block_scale are ignored (may be NULL);
 *          or NQ_MODE_MXFP8: q = (M, H) bytes of E4M3FN codes, block_scale =
 *          (M, H/32) bytes of E8M0 scale codes, both row-major; H % 32 == 0
 *          (NQ_EUNSUPPORTED otherwise); scale is ignored (may be NULL).
 *
 * Other arguments, layouts and errors as for nq_gemma_add_rms_norm_quant,
 * which equals this call with norm = NQ_NORM_GEMMA.
 */
nq_status nq_add_rms_norm_quant(const void *x, void *residual, const void *weight, float eps,
                                const float *scale, int64_t M, int64_t H, int dtype, int norm,
                                int mode, int write_y, void *q, void *block_scale, void *y,
                                void *stream);

/*
 * nq_quant_fp8_static / nq_quant_nvfp4 -- the standalone quant kernels of
 * the unfused chain that the `fused_norm_quant` module docstring says the
 * fused kernel replaces (an add + Gemma RMSNorm kernel, then a separate
 * static-FP8 or NVFP4 quant kernel using identical scale math).  y is an (M, H)
 * activation of `dtype`, row-major contiguous; the codes, block scales,
 * rounding and layout are exactly the fused op's quant step.
 *
 *   nq_quant_fp8_static: scale = DEVICE pointer to the static per-tensor
 *     scale; q = (M, H) E4M3FN bytes.  Any H >= 1.
 *   nq_quant_nvfp4: global_scale = DEVICE pointer to the NVFP4 global scale;
 *     q = (M, H/2) packed E2M1 bytes; block_scale = nq_block_scale_bytes(M, H)
 *     bytes, 128x4-tiled, rows >= M left as they were.  H % 16 == 0
 *     (NQ_EUNSUPPORTED otherwise); a partial last 4-column tile (H % 64 != 0)
 *     keeps its unused columns untouched.
 *
 * M == 0 returns NQ_OK without launching.
 */
nq_status nq_quant_fp8_static(const void *y, const float *scale, int64_t M, int64_t H, int dtype,
                              void *q, void *stream);
nq_status nq_quant_nvfp4(const void *y, const float *global_scale, int64_t M, int64_t H, int dtype,
                         void *q, void *block_scale, void *stream);

/*
 * nq_quant_mxfp8 -- standalone MXFP8 quant of an (M, H) activation y of
 * `dtype` (row-major contiguous), exactly the MXFP8 step of
 * nq_add_rms_norm_quant: q = (M, H) E4M3FN bytes, scales = (M, H/32) E8M0
 * bytes, both row-major.  H % 32 == 0 (NQ_EUNSUPPORTED otherwise); M == 0
 * returns NQ_OK without launching.
 */
nq_status nq_quant_mxfp8(const void *y, int64_t M, int64_t H, int dtype, void *q, void *scales,
                         void *stream);

/*
 * nq_gemm_mxfp8 / nq_gemm_fp8_static -- the consumer linear of the quantized
 * activation: out[M, N] = dq(a) * dq(b)^T, rounded to bf16, where a is the
 * (M, K) activation code matrix this library writes and b the (N, K) weight
 * codes in the same format, both row-major (K-contiguous).  This is the
 * pre-quantized input path of the quantized linears on the PR conversation
 * page: the linear takes the activation already quantized instead of
 * quantizing it again.
 *
 *   nq_gemm_mxfp8: a, b = E4M3FN codes; a_scales (M, K/32), b_scales
 *     (N, K/32) = E8M0 codes, row-major (the MXFP8 mode's layout);
 *     dq(x)[r, k] = E4M3(x[r, k]) * 2^(scale[r, k/32] - 127).
 *   nq_gemm_fp8_static: a, b = E4M3FN codes; a_scale, b_scale = DEVICE
 *     pointers to one fp32 each (the static FP8 mode's scale, and the
 *     weight's); dq(x) = E4M3(x) * scale.
 *   out: (M, N) bf16, row-major, round to nearest even of the fp32
 *     accumulation; must not overlap any input.
 *   M, N >= 0 (either 0: NQ_OK, nothing launched); K > 0 with K % 32 == 0
 *     (NQ_EUNSUPPORTED otherwise); a and b 16-byte aligned, out 2-byte
 *     aligned, the static scales 4-byte aligned (NQ_EINVAL otherwise).
 *
 * Accumulation: the block-scaled MFMA of gfx950 in fp32 accumulators; the
 * MFMA's internal sum of its 64 products is not an IEEE fp32 sum (measured
 * relative error up to ~2^-12 of sum |a b| per instruction).
 */
nq_status nq_gemm_mxfp8(const void *a, const void *a_scales, const void *b, const void *b_scales,
                        int64_t M, int64_t N, int64_t K, void *out, void *stream);
nq_status nq_gemm_fp8_static(const void *a, const float *a_scale, const void *b,
                             const float *b_scale, int64_t M, int64_t N, int64_t K, void *out,
                             void *stream);

/*
 * nq_gemm_nvfp4 -- the consumer linear of the NVFP4 output: out[M, N] =
 * dq(a) * dq(b)^T rounded to bf16, a the (M, K/2) packed E2M1 codes this
 * library writes (element 2j in the low nibble of byte j) and b the weight's
 * (N, K/2) codes in the same format; a_scales / b_scales the 128x4-tiled
 * E4M3FN block-scale buffers of nq_block_scale_bytes(M, K) /
 * nq_block_scale_bytes(N, K) bytes (the NVFP4 mode's layout: one scale per
 * 16 elements); a_gs / b_gs DEVICE pointers to the fp32 global scale each
 * operand was quantized with (the op's `scale` in NVFP4 mode).
 *   dq(x)[r, k] = E2M1(code) * E4M3(scale[r, k/16]) / gs.
 * The products are exact in fp32 (each dequantized value has at most 5
 * significant bits and lies in [2^-10, 2688] in magnitude, or is 0); the
 * sum is accumulated in fp32 and multiplied by 1 / (gs_a gs_b) before the
 * rounding to bf16.  Scale bytes of rows >= M (>= N) are read (they share
 * 512-byte tiles with real rows) but only reach outputs that are not
 * written.
 *   M, N >= 0 (either 0: NQ_OK, nothing launched); K > 0 with K % 64 == 0
 *   (NQ_EUNSUPPORTED otherwise); a, b and both scale buffers 16-byte
 *   aligned, out 2-byte aligned, a_gs and b_gs 4-byte aligned, out
 *   overlapping no input (NQ_EINVAL otherwise).
 */
nq_status nq_gemm_nvfp4(const void *a, const void *a_scales, const float *a_gs, const void *b,
                        const void *b_scales, const float *b_gs, int64_t M, int64_t N, int64_t K, void *out,
                        void *stream);

/*
 * nq_gemma_add_rms_norm_quant_gemm_fp8 -- a decode step: the op in static
 * FP8 mode on a few token rows and its consumer linear.  The
 * `fused_norm_quant` page overlaps the consumer GEMM's launch with the op at
 * small batches (its launch comment: an early trigger, ~2% at up to 128
 * rows).  Here, for M <= 3, the step is one launch: every GEMM workgroup
 * fetches its weight tile while it forms the rows' norm and FP8 codes
 * itself, so no second launch waits on the first.  For 4 <= M <= 8 the
 * redundant per-workgroup norm costs more than a launch, and the call runs
 * the op and the decode GEMM as two launches on the stream.
 *
 *   x, weight, eps, scale, M, H, dtype, write_y, q, y
 *              as nq_gemma_add_rms_norm_quant in NQ_MODE_FP8_STATIC; the
 *              results (q, y, the updated residual) are bit-for-bit those
 *              of that call.
 *   residual   (M, H) dtype or NULL, read only;
 *   residual_out (M, H) dtype, required with residual: x + residual
 *              (not in place: the launch's workgroups read the residual
 *              while one of them writes the result).
 *   b, b_scale the linear's weight: (N, H) E4M3FN codes, row-major, and its
 *              static fp32 scale (DEVICE pointer).
 *   N          output features >= 1.
 *   out        (M, N) bf16 = dq(q) dq(b)^T: bit-for-bit the result of
 *              nq_gemm_fp8_static(q, scale, b, b_scale) for 4 <= M <= 8, and
 *              for M <= 3 where that call runs its 32 x 16 decode tiles
 *              (H 2048 or 4096, N < 6144); elsewhere within that call's
 *              error bound (another K split).
 *
 * Shapes: 1 <= M <= 8 and H in {1024, 2048, 4096}; other M, H and N == 0
 * return NQ_EUNSUPPORTED (run the op and the GEMM as two calls); M == 0
 * returns NQ_OK without launching.  x, residual, residual_out, weight, y and
 * b 16-byte aligned, q 8-byte, out 2-byte, the scales 4-byte; outputs
 * (residual_out, q, y, out) overlap nothing (NQ_EINVAL otherwise, nothing
 * launched).
 */
nq_status nq_gemma_add_rms_norm_quant_gemm_fp8(const void *x, const void *residual, void *residual_out,
                                               const void *weight, float eps, const float *scale, int64_t M,
                                               int64_t H, int dtype, int write_y, void *q, void *y, const void *b,
                                               const float *b_scale, int64_t N, void *out, void *stream);

/* Size in bytes of the NVFP4 block-scale buffer:
 * round_up(M, 128) * round_up(H / 16, 4) (the wrapper's allocation on the
 * `fused_norm_quant` page).  0 for M <= 0, H < 16, or sizes the entry points
 * reject (H > 2^30 or M * H > 2^60). */
size_t nq_block_scale_bytes(int64_t M, int64_t H);

/* Static description of a status code; never NULL. */
const char *nq_status_string(int status);

/* NQ_ABI_VERSION of the loaded library. */
int nq_abi_version(void);

/*
 * nq_convert_probe -- diagnostic: runs the fused kernel's own device
 * conversion routines on n 32-bit input patterns, so that tests can sweep
 * them (every rounding tie and its neighbours, every 16-bit input) against
 * an independent encoder.
 *
 *   in   device buffer of n uint32 patterns
 *   kind 0: E4M3FN saturating encode of the fp32 pattern -> 1 byte each
 *   kind 1: E2M1 saturating encode of the fp32 pattern   -> 1 byte each
 *           (code in the low nibble)
 *   kind 2: bf16 round-to-nearest-even of the fp32 pattern -> 2 bytes each
 *   kind 3: fp16 round-to-nearest-even of the fp32 pattern -> 2 bytes each
 *   kind 4: static FP8 quant of bf16 y = low 16 bits of the pattern with
 *           scale `param` (the E4M3FN(y / scale) step) -> 1 byte each
 *   kind 5: kind 4 for fp16 y
 *   kind 6: NVFP4 block-scale code of amax = fp32 pattern with global scale
 *           `param` -> 1 byte each (exact for amax values a bf16 or an
 *           fp16 holds, the only ones the kernels pass)
 *   kind 7: MXFP8 E8M0 scale code of amax = |fp32 pattern| -> 1 byte each
 *   kind 8: MXFP8 element code of the fp32 pattern in a block whose E8M0
 *           scale code is `param` (an integer in [0, 247], else
 *           NQ_EINVAL) -> 1 byte each
 *   kind 9: NVFP4 element code of bf16 y = bits 0..15 of the pattern in a
 *           block whose E4M3FN scale code is bits 16..23, global scale
 *           `param` (the E2M1(y * gs / decode(S)) step) -> 1 byte each
 *           (code in the low nibble)
 *   kind 10: kind 4 through the vector routine the kernels use on 8-element
 *           chunks: patterns 8j .. 8j + 7 form one chunk (n % 8 == 0, else
 *           NQ_EINVAL) -> 1 byte each
 *   kind 11: kind 10 for fp16 y
 *   out  device buffer of n (kinds 0, 1, 4..11) or 2n (kinds 2, 3) bytes.
 *   n    in [0, 2^31).
 */
nq_status nq_convert_probe(int kind, const void *in, int64_t n, float param, void *out,
                           void *stream);

/*
 * nq_traffic_probe -- diagnostic: a kernel with the op's access structure
 * and none of its arithmetic, to measure the bandwidth a launch that moves
 * the op's bytes can reach (the practical ceiling the op's figures are
 * compared with).  Per row, every thread loads its 16-byte chunks (index
 * thread, thread + threads, ...) of each read stream with non-temporal
 * loads, folds them into one value and stores that value to its chunks of
 * each write stream with non-temporal stores.
 *
 *   src, src_row_bytes, nsrc   host arrays: 1 or 2 device read streams of
 *                              rows * src_row_bytes[i] bytes;
 *   dst, dst_row_bytes, ndst   host arrays: 0..4 device write streams of
 *                              rows * dst_row_bytes[i] bytes;
 *   rows                       >= 0 (0: NQ_OK, nothing launched);
 *   threads                    workgroup size, a multiple of 64 in [64, 1024];
 *   grid                       0: one workgroup per row; else that many
 *                              workgroups taking rows round-robin;
 *   flags                      NQ_PROBE_PREFETCH: issue the next row's loads
 *                              before the current row's stores;
 *                              NQ_PROBE_TILED_SCALES: the last write stream
 *                              holds one byte per 16 elements in the 128x4-
 *                              tiled NVFP4 block-scale layout (byte of block b
 *                              of row m at the offset nq_gemma_add_rms_norm_quant
 *                              stores it, with row_bytes / 4 four-block
 *                              tiles per 128 rows), stored one byte at a
 *                              time as the op stores its scales, and rows go
 *                              to workgroups in the op's NVFP4 row order;
 *                              rows must be a multiple of 128.
 * Row bytes must be positive multiples of 16 (a read row at most
 * 64 * threads bytes), pointers 16-byte aligned, and no write stream may
 * overlap another stream (NQ_EINVAL otherwise, as for any other flag bit).
 * The written bytes are meaningless.
 */
#define NQ_PROBE_PREFETCH 1
#define NQ_PROBE_TILED_SCALES 2
nq_status nq_traffic_probe(const void *const *src, const int64_t *src_row_bytes, int nsrc,
                           void *const *dst, const int64_t *dst_row_bytes, int ndst, int64_t rows,
                           int threads, int grid, int flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMMA_NORM_QUANT_H */
