// Fused residual-add + Gemma RMSNorm + FP8 / NVFP4 activation quant for
// MI355X (gfx950), behind the C ABI declared in include/gemma_norm_quant.h.
//
// The operation is `gemma_add_rms_norm_quant` on the `fused_norm_quant` page:
// residual <- x + residual (rounded to x's dtype), y = h * rsqrt(mean(h^2) +
// eps) * (1 + w) rounded to x's dtype, then static FP8 E4M3 codes of y/scale,
// or NVFP4: E2M1 codes with one E4M3 scale per 16 elements in the 128x4-tiled
// layout.  The page computes the codes from the rounded y so that they equal
// the unfused chain; this file does the same.
//
// Design (memory-bound; no MFMA -- nothing here is a contraction):
//  * One workgroup per row, grid = M (measured faster than a persistent grid
//    on this chip: more independent rows in flight and no row loop).  A
//    thread owns 8-element chunks (16 bytes) at chunk index tid, tid + nthr,
//    ..., so every load and store instruction of a wave covers contiguous
//    memory: 1 KB of x / residual / y, 512 B of FP8 codes, 256 B of FP4 codes.
//    1, 2 or 4 chunks per thread (H <= 4096, <= 16384, <= 32768).
//  * x and residual are streamed with non-temporal loads, all outputs with
//    non-temporal stores; the weight is a plain (L2-cached) load.  All loads
//    of a row are issued before the first wait.
//  * Sum of squares: fp32 FMA chain per thread, DPP butterfly inside each
//    16-lane row plus readlane across rows, one LDS slot per wave, one
//    barrier per row.
//  * An NVFP4 block (16 elements) is the chunk pair held by two adjacent
//    lanes; the block amax is combined with a DPP lane swap and the even lane
//    stores the block's scale byte at its 128x4-tiled offset.  NVFP4 rows are
//    assigned to workgroups so that each 128-row scale tile is written
//    through a single XCD.
//  * The per-element quant arithmetic is IEEE fp32 (correctly rounded
//    division, no contraction: the file is built with -ffp-contract=off) and
//    the format conversions are the gfx950 hardware ones: v_cvt_pk_bf16_f32 /
//    v_cvt_f16_f32 (RNE), v_cvt_pk_fp8_f32 (OCP E4M3, RNE) after an explicit
//    clamp to +-448, v_cvt_scalef32_pk_fp4_f32 with unit scale after a clamp
//    to +-6.  Their semantics are checked exhaustively against the CPU oracle
//    through nq_convert_probe.
//  * H <= 512: several rows per wavefront (fused_rows_small), reduced inside
//    lane groups with DPP, no barrier.
//  * Shapes or pointers the vector path cannot take (H % 16 != 0, H > 32768,
//    unaligned views) go to a scalar kernel with the same arithmetic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemma_norm_quant.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kVec = 8;           // elements per thread chunk (16 bytes)
constexpr int kBlock = 16;        // elements per NVFP4 block scale
constexpr int kWave = 64;
constexpr int kMaxThreads = 1024;
constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// ----------------------------------------------------------------------------
// Activation dtypes: unpack two values from a 32-bit word, pack two fp32
// values with round-to-nearest-even.
struct Bf16 {
  static __device__ __forceinline__ float lo(uint32_t p) { return __uint_as_float(p << 16); }
  static __device__ __forceinline__ float hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

struct Fp16 {
  static __device__ __forceinline__ float lo(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};

// ----------------------------------------------------------------------------
// Quant-side encoders (shared by the kernels and the probe).

__device__ __forceinline__ float clampf(float v, float lim) {
  return __builtin_amdgcn_fmed3f(v, -lim, lim);
}

// Four E4M3FN codes (saturating, RNE) packed little-endian into a word.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf(a, kE4M3Max), clampf(b, kE4M3Max), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf(c, kE4M3Max), clampf(d, kE4M3Max), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3_one(float a) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clampf(a, kE4M3Max), 0.0f, 0, false) & 0xffu;
}

// Eight E2M1 codes, element 2k in the low nibble of byte k.  The gfx950
// conversion rounds to nearest even and saturates out-of-range magnitudes
// (including infinities) to 6 by itself, so no clamp precedes it; the
// exhaustive probe tests check it against clamp-then-round.
__device__ __forceinline__ uint32_t e2m1x8(const float *v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// fl32(y / s), correctly rounded, from r = fl32(1 / s) (one IEEE division
// per thread instead of one per element).  q0 = fl(y * r) lies within 1.5
// ulp of y / s; a correction step q + (y - q*s) * r (FMA, one rounding)
// brings it within 1 ulp, and from there one more step gives the correctly
// rounded quotient (Markstein's theorem: reciprocal within half an ulp,
// quotient within one ulp, exact remainder).  The remainder is exact for
// |y| >= 2^-103, i.e. for every scale >= 2^-90 wherever the FP8 code is not
// zero.  Quotients beyond +-1024 saturate to +-448 either way; clamping them
// between steps keeps every intermediate finite.  The remainder is formed as
// q*s - y and subtracted, so a zero quotient keeps the sign of y.
__device__ __forceinline__ float div_by_scale(float y, float s, float r) {
  float q = clampf(y * r, 1024.0f);
  q = clampf(__builtin_fmaf(-__builtin_fmaf(q, s, -y), r, q), 1024.0f);
  return __builtin_fmaf(-__builtin_fmaf(q, s, -y), r, q);
}

// NVFP4 block scale: S = E4M3(min(gs * (amax / 6), 448)).
__device__ __forceinline__ uint32_t nvfp4_scale_code(float amax, float gs) {
  const float t = amax / kE2M1Max;
  const float u = fminf(gs * t, kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, 0, false) & 0xffu;
}

// Element multiplier o = gs / decode(S), 0 for a zero scale.
__device__ __forceinline__ float nvfp4_elem_scale(uint32_t s_code, float gs) {
  const float sigma = __builtin_amdgcn_cvt_f32_fp8((int)s_code, 0);
  return sigma == 0.0f ? 0.0f : gs / sigma;
}

// Byte offset of block scale (row m, block b) in the 128x4-tiled layout;
// ktiles = round_up(H/16, 4) / 4.
__device__ __forceinline__ size_t swz128x4(int64_t m, int b, int ktiles) {
  return ((size_t)(m >> 7) * (size_t)ktiles + (size_t)(b >> 2)) * 512u + (size_t)(m & 31) * 16u +
         (size_t)((m >> 5) & 3) * 4u + (size_t)(b & 3);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

// Value of the neighbouring lane (lane ^ 1): DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ float dpp_swap_adjacent(float v) { return dpp<0xB1>(v); }

// Sum over the 64 lanes of a wave (all lanes active), returned to every lane:
// DPP exchanges inside each 16-lane row (lane ^ 1, lane ^ 2, 8-lane mirror,
// 16-lane mirror), then the four row totals via readlane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  const int b = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// Workgroup -> row for NVFP4.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8).  Inside every full span of 1024
// rows, XCD x takes the whole 128-row tile x, so the 32 rows that share each
// 128-byte line of the 128x4-tiled scales write it through one XCD's L2 and
// the line reaches HBM once (measured: scale writes drop from ~2x to 1x,
// 5% faster at M = 8192).  Rows of a ragged last span map to themselves.
__device__ __forceinline__ int64_t nvfp4_row_of_block(int64_t b, int64_t M) {
  if ((((b >> 10) + 1) << 10) > M) return b;
  const int64_t lo = b & 1023;
  return ((b >> 10) << 10) + ((lo & 7) << 7) + (lo >> 3);
}

// ----------------------------------------------------------------------------
// Vector kernel.  A workgroup normalises one row (grid = M; the row loop only
// runs more than once if M exceeds the grid limit).  A chunk is 8 elements
// (16 bytes of x's dtype); thread t owns chunks t, t + nthr, ... (CPT of
// them), so each load/store instruction of a wave covers 1 KB of contiguous
// 16-bit data.  An NVFP4 block is the chunk pair (2j, 2j+1), held by two
// adjacent lanes of one wave; their amax is combined with a DPP lane swap.
template <class D, bool NVFP4, bool HAS_RES, bool WRITE_Y, int CPT>
__global__ void __launch_bounds__(kMaxThreads)
fused_rows(const u32x4 *__restrict__ x, u32x4 *__restrict__ res, const u32x4 *__restrict__ w,
           const float *__restrict__ scale_ptr, float eps, int64_t M, int nchunk,
           uint8_t *__restrict__ q, uint8_t *__restrict__ bs, u32x4 *__restrict__ y, int ktiles) {
  __shared__ float partial[2][kMaxThreads / kWave];
  const unsigned tid = threadIdx.x;
  const unsigned nthr = blockDim.x;
  const unsigned nch = (unsigned)nchunk;
  const int nwaves = nthr / kWave;
  const float Hf = (float)(nchunk * kVec);
  int parity = 0;
  for (int64_t blk = blockIdx.x; blk < M; blk += gridDim.x, parity ^= 1) {
    const int64_t row = NVFP4 ? nvfp4_row_of_block(blk, M) : blk;
    const size_t rbase = (size_t)row * (size_t)nchunk;
    const u32x4 *__restrict__ xr = x + rbase;
    u32x4 *__restrict__ rr = res + rbase;
    u32x4 *__restrict__ yr = y + rbase;
    // All loads first: x and residual stream from HBM (non-temporal), the
    // weight and the scale come from L2.  The scale's reciprocal is formed
    // while the row loads are in flight.
    u32x4 xa[CPT], ra[CPT], wa[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) {
        xa[c] = __builtin_nontemporal_load(&xr[ch]);
        if constexpr (HAS_RES) ra[c] = __builtin_nontemporal_load(&rr[ch]);
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) wa[c] = w[ch];
    }
    const float s = *scale_ptr;
    const float r_s = NVFP4 ? 0.0f : 1.0f / s;
    // h = RN(x + r), written back; sum of squares of the rounded h.
    uint32_t hb[CPT][4];
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) {
        if constexpr (HAS_RES) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            hb[c][k] = D::pack(D::lo(xa[c][k]) + D::lo(ra[c][k]), D::hi(xa[c][k]) + D::hi(ra[c][k]));
          const u32x4 o = {hb[c][0], hb[c][1], hb[c][2], hb[c][3]};
          __builtin_nontemporal_store(o, &rr[ch]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) hb[c][k] = xa[c][k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float a = D::lo(hb[c][k]), b = D::hi(hb[c][k]);
          ss = __builtin_fmaf(a, a, ss);
          ss = __builtin_fmaf(b, b, ss);
        }
      }
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) partial[parity][tid / kWave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int i = 0; i < nwaves; ++i) tot += partial[parity][i];
    const float rstd = 1.0f / __builtin_sqrtf(tot / Hf + eps);

#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const unsigned ch = tid + c * nthr;
      if (ch < nch) {
        // y = RN(t * (1 + w)) with t = h * rstd, formed as fma(t, w, t): one
        // rounding of the exact t * (1 + w).  The quant reads the rounded y.
        float yv[kVec];
        uint32_t yb[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float ta = D::lo(hb[c][k]) * rstd, tb = D::hi(hb[c][k]) * rstd;
          const float a = __builtin_fmaf(ta, D::lo(wa[c][k]), ta);
          const float b = __builtin_fmaf(tb, D::hi(wa[c][k]), tb);
          yb[k] = D::pack(a, b);
          yv[2 * k] = D::lo(yb[k]);
          yv[2 * k + 1] = D::hi(yb[k]);
        }
        if constexpr (WRITE_Y) {
          const u32x4 o = {yb[0], yb[1], yb[2], yb[3]};
          __builtin_nontemporal_store(o, &yr[ch]);
        }
        if constexpr (NVFP4) {
          float amax = 0.0f;
#pragma unroll
          for (int k = 0; k < kVec; ++k) amax = fmaxf(amax, fabsf(yv[k]));
          amax = fmaxf(amax, dpp_swap_adjacent(amax));
          const uint32_t sc = nvfp4_scale_code(amax, s);
          const float o = nvfp4_elem_scale(sc, s);
          float v[kVec];
#pragma unroll
          for (int k = 0; k < kVec; ++k) v[k] = yv[k] * o;
          uint32_t *qrow = reinterpret_cast<uint32_t *>(q + (size_t)row * (size_t)nchunk * 4);
          __builtin_nontemporal_store(e2m1x8(v), &qrow[ch]);
          if ((ch & 1) == 0) bs[swz128x4(row, ch >> 1, ktiles)] = (uint8_t)sc;
        } else {
          float v[kVec];
#pragma unroll
          for (int k = 0; k < kVec; ++k) v[k] = div_by_scale(yv[k], s, r_s);
          const u32x2 packed = {e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7])};
          u32x2 *qrow = reinterpret_cast<u32x2 *>(q + (size_t)row * (size_t)nchunk * 8);
          __builtin_nontemporal_store(packed, &qrow[ch]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Small-H kernel (H <= 512): several rows per wavefront.  A row takes LPR
// lanes (the power of two >= H/8, one 8-element chunk per lane), a wave holds
// 64/LPR rows and a 256-thread workgroup 4 times as many.  The row sum of
// squares is a DPP/shuffle reduction inside the LPR-lane group, so waves
// never wait on each other: no LDS, no barrier.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPR >= 2) v += dpp<0xB1>(v);    // lane ^ 1
  if constexpr (LPR >= 4) v += dpp<0x4E>(v);    // lane ^ 2
  if constexpr (LPR >= 8) v += dpp<0x141>(v);   // mirror inside 8 lanes
  if constexpr (LPR >= 16) v += dpp<0x140>(v);  // mirror inside 16 lanes
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

constexpr int kSmallThreads = 256;

template <class D, bool NVFP4, bool HAS_RES, bool WRITE_Y, int LPR>
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
  const float s = *scale_ptr;
  const float r_s = NVFP4 ? 0.0f : 1.0f / s;
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
  const float rstd = 1.0f / __builtin_sqrtf(ss / (float)(nchunk * kVec) + eps);
  float yv[kVec];
  uint32_t yb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float ta = D::lo(hb[k]) * rstd, tb = D::hi(hb[k]) * rstd;
    yb[k] = D::pack(__builtin_fmaf(ta, D::lo(wa[k]), ta), __builtin_fmaf(tb, D::hi(wa[k]), tb));
    yv[2 * k] = D::lo(yb[k]);
    yv[2 * k + 1] = D::hi(yb[k]);
  }
  if constexpr (WRITE_Y) {
    if (active) {
      const u32x4 o = {yb[0], yb[1], yb[2], yb[3]};
      __builtin_nontemporal_store(o, &y[rbase + ch]);
    }
  }
  if constexpr (NVFP4) {
    // H % 64 == 0, so a row's lanes pair up into whole blocks and inactive
    // lanes pair only with inactive lanes.
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < kVec; ++k) amax = fmaxf(amax, fabsf(yv[k]));
    amax = fmaxf(amax, dpp_swap_adjacent(amax));
    const uint32_t sc = nvfp4_scale_code(amax, s);
    const float o = nvfp4_elem_scale(sc, s);
    float v[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) v[k] = yv[k] * o;
    const uint32_t packed = e2m1x8(v);
    if (active) {
      uint32_t *qrow = reinterpret_cast<uint32_t *>(q + (size_t)row * (size_t)nchunk * 4);
      __builtin_nontemporal_store(packed, &qrow[ch]);
      if ((ch & 1) == 0) bs[swz128x4(row, ch >> 1, ktiles)] = (uint8_t)sc;
    }
  } else {
    float v[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) v[k] = div_by_scale(yv[k], s, r_s);
    const u32x2 packed = {e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7])};
    if (active) {
      u32x2 *qrow = reinterpret_cast<u32x2 *>(q + (size_t)row * (size_t)nchunk * 8);
      __builtin_nontemporal_store(packed, &qrow[ch]);
    }
  }
}

// ----------------------------------------------------------------------------
// Scalar kernel for any H and any alignment: same arithmetic, element loads.
template <class D, bool NVFP4, bool HAS_RES, bool WRITE_Y>
__global__ void __launch_bounds__(256)
fused_rows_scalar(const uint16_t *__restrict__ x, uint16_t *__restrict__ res,
                  const uint16_t *__restrict__ w, const float *__restrict__ scale_ptr, float eps,
                  int64_t M, int H, uint8_t *__restrict__ q, uint8_t *__restrict__ bs,
                  uint16_t *__restrict__ y, int ktiles) {
  __shared__ float partial[2][256 / kWave];
  const int tid = threadIdx.x;
  const int nwaves = blockDim.x / kWave;
  const float s = *scale_ptr;
  const float r_s = 1.0f / s;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < M; row += gridDim.x, parity ^= 1) {
    const size_t rb = (size_t)row * (size_t)H;
    float ss = 0.0f;
    for (int j = tid; j < H; j += blockDim.x) {
      uint32_t h = x[rb + j];
      if constexpr (HAS_RES) {
        h = D::pack(D::lo(h) + D::lo(res[rb + j]), 0.0f) & 0xffffu;
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
    const float rstd = 1.0f / __builtin_sqrtf(tot / (float)H + eps);
    const uint16_t *hsrc = HAS_RES ? res : x;
    if constexpr (NVFP4) {
      // Blocks of 16 read h written by other threads before the barrier.
      const int nb = H / kBlock;
      for (int b = tid; b < nb; b += blockDim.x) {
        float yv[kBlock];
        for (int k = 0; k < kBlock; ++k) {
          const int j = b * kBlock + k;
          const float t = D::lo(hsrc[rb + j]) * rstd;
          const float yy = __builtin_fmaf(t, D::lo(w[j]), t);
          const uint32_t yq = D::pack(yy, 0.0f) & 0xffffu;
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
    } else {
      for (int j = tid; j < H; j += blockDim.x) {
        const float t = D::lo(hsrc[rb + j]) * rstd;
          const float yy = __builtin_fmaf(t, D::lo(w[j]), t);
        const uint32_t yq = D::pack(yy, 0.0f) & 0xffffu;
        if constexpr (WRITE_Y) y[rb + j] = (uint16_t)yq;
        q[rb + j] = (uint8_t)e4m3_one(div_by_scale(D::lo(yq), s, r_s));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Conversion probe (diagnostics): the same device routines on bit patterns.
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
    default: break;
  }
}

// ----------------------------------------------------------------------------
// Host side.

template <class D, bool NV, bool RES, bool WY, int CPT>
hipError_t launch_vec(dim3 grid, dim3 block, hipStream_t st, const void *x, void *res, const void *w,
                      const float *scale, float eps, int64_t M, int nchunk, void *q, void *bs,
                      void *y, int ktiles) {
  hipLaunchKernelGGL((fused_rows<D, NV, RES, WY, CPT>), grid, block, 0, st,
                     (const u32x4 *)x, (u32x4 *)res, (const u32x4 *)w, scale, eps, M, nchunk,
                     (uint8_t *)q, (uint8_t *)bs, (u32x4 *)y, ktiles);
  return hipGetLastError();
}

template <class D, bool NV, bool RES, bool WY, int LPR>
hipError_t launch_small(hipStream_t st, const void *x, void *res, const void *w,
                        const float *scale, float eps, int64_t M, int nchunk, void *q, void *bs,
                        void *y, int ktiles) {
  constexpr int64_t rows_per_wg = kSmallThreads / LPR;
  const int64_t blocks = (M + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((fused_rows_small<D, NV, RES, WY, LPR>), dim3((unsigned)blocks),
                     dim3(kSmallThreads), 0, st, (const u32x4 *)x, (u32x4 *)res, (const u32x4 *)w,
                     scale, eps, M, nchunk, (uint8_t *)q, (uint8_t *)bs, (u32x4 *)y, ktiles);
  return hipGetLastError();
}

template <class D, bool NV, bool RES, bool WY>
hipError_t launch_scalar(dim3 grid, hipStream_t st, const void *x, void *res, const void *w,
                         const float *scale, float eps, int64_t M, int H, void *q, void *bs,
                         void *y, int ktiles) {
  hipLaunchKernelGGL((fused_rows_scalar<D, NV, RES, WY>), grid, dim3(256), 0, st,
                     (const uint16_t *)x, (uint16_t *)res, (const uint16_t *)w, scale, eps, M, H,
                     (uint8_t *)q, (uint8_t *)bs, (uint16_t *)y, ktiles);
  return hipGetLastError();
}

struct Args {
  const void *x;
  void *res;
  const void *w;
  const float *scale;
  float eps;
  int64_t M;
  int64_t H;
  void *q;
  void *bs;
  void *y;
  hipStream_t st;
};

constexpr int64_t kMaxGrid = ((int64_t)1 << 31) - 1;

// Chunks per thread for the vector kernel: one 8-element chunk per thread up
// to H = 4096 (short per-thread chains for latency), two up to H = 16384,
// four up to H = 32768 (at most 1024 threads per workgroup).
int chunks_per_thread(int64_t H) {
  const int64_t nchunk = H / kVec;
  if (H <= 4096) return 1;
  if (nchunk <= 2 * kMaxThreads) return 2;
  return 4;
}

template <class D, bool NV, bool RES, bool WY>
hipError_t run(const Args &a) {
  const int ktiles = (int)(((a.H / kBlock) + 3) / 4);
  auto aligned = [](const void *p, uintptr_t n) { return p == nullptr || ((uintptr_t)p % n) == 0; };
  const bool vec = (a.H % kBlock == 0) && (a.H / kVec) <= 4 * kMaxThreads && aligned(a.x, 16) &&
                   aligned(a.res, 16) && aligned(a.w, 16) && aligned(a.y, 16) &&
                   aligned(a.q, NV ? 4 : 8);
  const dim3 grid((unsigned)(a.M < kMaxGrid ? a.M : kMaxGrid));
  if (vec && a.H <= 512 && a.M <= kMaxGrid) {
    // Several rows per wave; lanes per row = the power of two >= H/8.
    const int nchunk = (int)(a.H / kVec);
    if (nchunk <= 2)
      return launch_small<D, NV, RES, WY, 2>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
    if (nchunk <= 4)
      return launch_small<D, NV, RES, WY, 4>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
    if (nchunk <= 8)
      return launch_small<D, NV, RES, WY, 8>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
    if (nchunk <= 16)
      return launch_small<D, NV, RES, WY, 16>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
    if (nchunk <= 32)
      return launch_small<D, NV, RES, WY, 32>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
    return launch_small<D, NV, RES, WY, 64>(a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, nchunk, a.q, a.bs, a.y, ktiles);
  }
  if (vec) {
    const int nchunk = (int)(a.H / kVec);
    const int cpt = chunks_per_thread(a.H);
    const int per_thread = (nchunk + cpt - 1) / cpt;
    const dim3 block(((per_thread + kWave - 1) / kWave) * kWave);
    if (cpt == 1)
      return launch_vec<D, NV, RES, WY, 1>(grid, block, a.st, a.x, a.res, a.w, a.scale, a.eps, a.M,
                                           nchunk, a.q, a.bs, a.y, ktiles);
    if (cpt == 2)
      return launch_vec<D, NV, RES, WY, 2>(grid, block, a.st, a.x, a.res, a.w, a.scale, a.eps, a.M,
                                           nchunk, a.q, a.bs, a.y, ktiles);
    return launch_vec<D, NV, RES, WY, 4>(grid, block, a.st, a.x, a.res, a.w, a.scale, a.eps, a.M,
                                         nchunk, a.q, a.bs, a.y, ktiles);
  }
  return launch_scalar<D, NV, RES, WY>(grid, a.st, a.x, a.res, a.w, a.scale, a.eps, a.M, (int)a.H,
                                       a.q, a.bs, a.y, ktiles);
}

template <class D, bool NV>
hipError_t run_res_y(const Args &a, bool res, bool wy) {
  if (res) return wy ? run<D, NV, true, true>(a) : run<D, NV, true, false>(a);
  return wy ? run<D, NV, false, true>(a) : run<D, NV, false, false>(a);
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x0 = (uintptr_t)a, x1 = x0 + na, y0 = (uintptr_t)b, y1 = y0 + nb;
  return x0 < y1 && y0 < x1;
}

}  // namespace

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

size_t nq_block_scale_bytes(int64_t M, int64_t H) {
  if (M <= 0 || H < kBlock) return 0;
  const int64_t rows = (M + 127) / 128 * 128;
  const int64_t cols = ((H / kBlock) + 3) / 4 * 4;
  return (size_t)rows * (size_t)cols;
}

nq_status nq_gemma_add_rms_norm_quant(const void *x, void *residual, const void *weight, float eps,
                                      const float *scale, int64_t M, int64_t H, int dtype,
                                      int mode, int write_y, void *q, void *block_scale, void *y,
                                      void *stream) {
  if (dtype != NQ_BF16 && dtype != NQ_FP16) return NQ_EINVAL;
  if (mode != NQ_MODE_FP8_STATIC && mode != NQ_MODE_NVFP4) return NQ_EINVAL;
  if (M < 0 || H <= 0 || H > (int64_t)1 << 30) return NQ_EINVAL;
  if (!x || !weight || !scale || !q) return NQ_EINVAL;
  const bool nv = mode == NQ_MODE_NVFP4;
  if (nv && !block_scale) return NQ_EINVAL;
  if (write_y && !y) return NQ_EINVAL;
  if (nv && H % 64 != 0) return NQ_EUNSUPPORTED;
  const size_t act = (size_t)M * (size_t)H * 2;
  const size_t qbytes = nv ? (size_t)M * (size_t)(H / 2) : (size_t)M * (size_t)H;
  const size_t bsbytes = nv ? nq_block_scale_bytes(M, H) : 0;
  if (residual == x) return NQ_EINVAL;
  if (overlaps(x, act, residual, act) || overlaps(q, qbytes, x, act) ||
      overlaps(q, qbytes, residual, act) || (write_y && (overlaps(y, act, x, act) ||
                                                          overlaps(y, act, residual, act) ||
                                                          overlaps(y, act, q, qbytes))) ||
      (nv && (overlaps(block_scale, bsbytes, x, act) || overlaps(block_scale, bsbytes, residual, act) ||
              overlaps(block_scale, bsbytes, q, qbytes) ||
              (write_y && overlaps(block_scale, bsbytes, y, act)))))
    return NQ_EINVAL;
  if (M == 0) return NQ_OK;

  Args a{x, residual, weight, scale, eps, M, H, q, nv ? block_scale : nullptr,
         write_y ? y : nullptr, (hipStream_t)stream};
  hipError_t e;
  const bool res = residual != nullptr, wy = write_y != 0;
  if (dtype == NQ_BF16)
    e = nv ? run_res_y<Bf16, true>(a, res, wy) : run_res_y<Bf16, false>(a, res, wy);
  else
    e = nv ? run_res_y<Fp16, true>(a, res, wy) : run_res_y<Fp16, false>(a, res, wy);
  return e == hipSuccess ? NQ_OK : NQ_EHIP;
}

nq_status nq_convert_probe(int kind, const void *in, int64_t n, float param, void *out,
                           void *stream) {
  if (kind < 0 || kind > 6 || n < 0 || n >= ((int64_t)1 << 31) || (n > 0 && (!out || !in)))
    return NQ_EINVAL;
  if (n == 0) return NQ_OK;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(convert_probe, dim3((unsigned)blocks), dim3(threads), 0, (hipStream_t)stream,
                     kind, (const uint32_t *)in, n, param, (uint8_t *)out);
  return hipGetLastError() == hipSuccess ? NQ_OK : NQ_EHIP;
}

}  // extern "C"
