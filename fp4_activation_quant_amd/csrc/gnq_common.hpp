// Device building blocks shared by every kernel of the library: activation
// dtypes, the FP8 / FP4 encoders, the correctly rounded division by the FP8
// scale, the NVFP4 and MXFP8 block-scale arithmetic, the 128x4 scale layout,
// DPP reductions, and the host-side argument block.
//
// The operation is `gemma_add_rms_norm_quant` on the `fused_norm_quant` page
// (and its unfused form: an add + Gemma RMSNorm kernel followed by a
// standalone static-FP8 or NVFP4 quant, which the page says the fused kernel
// matches code for code).  Format conversions are the gfx950 hardware
// instructions; the per-element arithmetic is IEEE fp32 with no contraction
// (the library is built with -ffp-contract=off and correctly rounded
// divide/sqrt).  The probe entry point of the C ABI runs these routines on
// arbitrary bit patterns so tests can check them exhaustively against the
// CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gnq_consts.hpp"
#include "gnq_launch.hpp"

namespace gnq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

// Output modes (values of nq_mode).
constexpr int kModeFp8 = 0;
constexpr int kModeNvfp4 = 1;
constexpr int kModeNone = 2;
constexpr int kModeMxfp8 = 3;

// Whether a mode reads the fp32 scale argument (MXFP8 derives its scales
// from the data; no quant has none).
constexpr bool mode_reads_scale(int mode) { return mode == kModeFp8 || mode == kModeNvfp4; }

// ----------------------------------------------------------------------------
// Activation dtypes: unpack two values from a 32-bit word, pack two fp32
// values with round-to-nearest-even.
struct Bf16 {
  static constexpr bool kF16 = false;
  static __device__ __forceinline__ float lo(uint32_t p) { return __uint_as_float(p << 16); }
  static __device__ __forceinline__ float hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
  // fl32(v * b + c), one rounding, for the low / high value v of p.
  static __device__ __forceinline__ float fma_lo(uint32_t p, float b, float c) { return __builtin_fmaf(lo(p), b, c); }
  static __device__ __forceinline__ float fma_hi(uint32_t p, float b, float c) { return __builtin_fmaf(hi(p), b, c); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  // One value rounded to bf16, in the low 16 bits (as Fp16::round1).
  static __device__ __forceinline__ uint32_t round1(float a) {
    asm("" : "+v"(a));
    return pack(a, 0.0f) & 0xffffu;
  }
};

struct Fp16 {
  static constexpr bool kF16 = true;
  static __device__ __forceinline__ float lo(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t p) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
  }
  // fl32(v * b + c), one rounding, for the low / high value v of p, with v
  // read from its half of p by v_fma_mix_f32 (whose widening of v is exact).
  // Written out because the compiler does not form the instruction where
  // the widening is shared with other uses of v.
  static __device__ __forceinline__ float fma_lo(uint32_t p, float b, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(p), "v"(b), "v"(c));
    return d;
  }
  static __device__ __forceinline__ float fma_hi(uint32_t p, float b, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(p), "v"(b), "v"(c));
    return d;
  }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  // One value rounded to fp16, in the low 16 bits.  The value passes an
  // empty asm first: without it the compiler folds a product feeding a lone
  // conversion into v_fma_mixlo_f16 with a +0 addend, which rounds the exact
  // product once (not to fp32, then to fp16) and turns a -0 product into +0.
  static __device__ __forceinline__ uint32_t round1(float a) {
    asm("" : "+v"(a));
    return pack(a, 0.0f) & 0xffffu;
  }
  // Both values of p clamped to [-L, L], L a non-negative fp16 held in both
  // halves of l2 (two packed instructions for two values).
  static __device__ __forceinline__ uint32_t clamp2(uint32_t p, uint32_t l2) {
    uint32_t t, r;
    asm("v_pk_max_f16 %0, %1, %2 neg_lo:[0,1] neg_hi:[0,1]" : "=v"(t) : "v"(p), "v"(l2));
    asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(t), "v"(l2));
    return r;
  }
};

// ----------------------------------------------------------------------------
// Quant-side encoders.

__device__ __forceinline__ float clampf(float v, float lim) {
  return __builtin_amdgcn_fmed3f(v, -lim, lim);
}

// Four E4M3FN codes packed little-endian into a word.  v_cvt_pk_fp8_f32
// rounds to nearest even but does not saturate (465 -> NaN), hence the clamp.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf(a, kE4M3Max), clampf(b, kE4M3Max), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clampf(c, kE4M3Max), clampf(d, kE4M3Max), w, true);
  return (uint32_t)w;
}

// e4m3x4 without the clamp: exact for |v| <= 464 (values in (448, 464]
// round to the saturated code, beyond 464 the conversion gives NaN).  (The first
// conversion's untouched half is overwritten by the second, so it starts
// from a's bits rather than a zero that would cost a move.)
__device__ __forceinline__ uint32_t e4m3x4_near(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
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
  // every byte of w is written below, so it may start from any bits
  uint32_t w = __builtin_bit_cast(uint32_t, v[0]);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// The quant step's per-tensor constants, formed once per thread: the
// scale s (FP8: the static scale; NVFP4: the global scale), r = fl32(1 / s)
// and, for FP8, the clamp bound lim = fl32(456 s) of div_by_scale.
struct QuantScale {
  float s, r, lim, nz;
  uint32_t lim2;   // static FP8: fl32(456 s) rounded to fp16, in both halves
  bool lim2_ok;    // 2^-22 <= s <= 143: lim2 is a finite normal fp16
  double r64;      // static FP8: RN64(1 / s)
};

__device__ __forceinline__ QuantScale quant_scale(float s, bool fp8);

// fl32(y / s), correctly rounded, from r = fl32(1 / s) (one IEEE division
// per thread instead of one per element).  q0 = fl(y * r) lies within 1.5
// ulp of y / s; a correction step q + (y - q*s) * r (FMA, one rounding)
// brings it within 1 ulp, and from there one more step gives the correctly
// rounded quotient (Markstein's theorem: reciprocal within half an ulp,
// quotient within one ulp, exact remainder).  The remainder is exact for
// |y| >= 2^-103, i.e. for every scale >= 2^-90 wherever the FP8 code is not
// zero.  y is first clamped to +-L, L = fl(456 s): a y beyond L has
// |y| / s > 455 and the saturated code, and so does +-L itself, whose
// quotient lies within 0.01 of 456.  So every quotient stays within +-464,
// where the conversion needs no clamp of its own (e4m3x4_near), and every
// intermediate stays finite (one clamp instead of one per step).  The
// remainder is formed as q*s - y and subtracted, so a zero quotient keeps
// the sign of y.  (A NaN y, outside the contract, clamps to -L.)
__device__ __forceinline__ float div_by_scale(float y, const QuantScale &d) {
  y = clampf(y, d.lim);
  float q = y * d.r;
  q = __builtin_fmaf(-__builtin_fmaf(q, d.s, -y), d.r, q);
  return __builtin_fmaf(-__builtin_fmaf(q, d.s, -y), d.r, q);
}

// fl32(y / s) for a y that a bf16 or an fp16 holds (at most 11
// significant bits), as RN32(RN64(y * RN64(1/s))): the double product is
// within 2^-52 relative of y / s (two roundings of 2^-53), while y / s is
// never within 2^-49 relative of a point halfway between two floats (that
// midpoint has a 25-bit odd significand m; y = Y 2^a, s = S 2^b with Y and
// S odd of at most 11 and 24 bits, so y - m 2^c s is a nonzero multiple of
// 2^min(a, b + c), at least 2^-49 of m S 2^(b + c)), so both round to the
// same float (quotients below 2^-126, where that spacing argument ends,
// take the code +-0 either way).  Five instructions per value with the two
// widenings, against
// six for div_by_scale's reciprocal and corrections (the fp64 multiply runs
// at the fp32 rate on this part).  Bit-identical to div_by_scale wherever
// both apply.  y clamped as in div_by_scale (the clamp bound L may have
// more bits than y, but its quotient lies next to 456, far from any code
// boundary, so its code is the saturated one either way).
__device__ __forceinline__ float div_by_scale_f64(float y, const QuantScale &d) {
  return (float)((double)y * d.r64);
}

// Static FP8 codes of one 8-element chunk of rounded y (four words of two
// activation-dtype values), little-endian.  fp16 y are clamped in pairs in
// their own format (lim2, the fp16 rounding of L: within (455.7 s,
// 456.3 s), so the argument of div_by_scale holds unchanged) where that
// bound is a finite normal fp16; other scales and bf16 y take the fp32
// clamp.
template <class D>
__device__ __forceinline__ u32x2 fp8_codes(const uint32_t (&yb)[4], const QuantScale &d) {
  float v[kVec];
  if constexpr (D::kF16) {
    if (d.lim2_ok) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t c = Fp16::clamp2(yb[k], d.lim2);
        v[2 * k] = div_by_scale_f64(Fp16::lo(c), d);
        v[2 * k + 1] = div_by_scale_f64(Fp16::hi(c), d);
      }
      return u32x2{e4m3x4_near(v[0], v[1], v[2], v[3]), e4m3x4_near(v[4], v[5], v[6], v[7])};
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = div_by_scale_f64(clampf(D::lo(yb[k]), d.lim), d);
    v[2 * k + 1] = div_by_scale_f64(clampf(D::hi(yb[k]), d.lim), d);
  }
  return u32x2{e4m3x4_near(v[0], v[1], v[2], v[3]), e4m3x4_near(v[4], v[5], v[6], v[7])};
}

// -0.0 in a register the optimizer cannot see into.  fma(a, b, -0) is the
// same single rounding of the exact product as a * b (signed zeros
// included); written with this addend it is not folded back into a
// multiply, so an fp16 operand is read straight from its packed half
// (v_fma_mix_f32) instead of being unpacked first.
__device__ __forceinline__ float opaque_neg_zero() {
  float z;
  asm("v_mov_b32 %0, 0x80000000" : "=v"(z));
  return z;
}

__device__ __forceinline__ QuantScale quant_scale(float s, bool fp8) {
  const float lim = fp8 ? 456.0f * s : 0.0f;
  return QuantScale{s, fp8 ? 1.0f / s : 0.0f, lim, opaque_neg_zero(), Fp16::pack(lim, lim),
                    fp8 && s >= 0x1p-22f && s <= 143.0f, fp8 ? 1.0 / (double)s : 0.0};
}

// fl32(y * o) for each value of a chunk (nz: opaque_neg_zero()).
template <class D>
__device__ __forceinline__ void scale_chunk(const uint32_t (&yb)[4], float o, float nz, float (&v)[kVec]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __builtin_fmaf(D::lo(yb[k]), o, nz);
    v[2 * k + 1] = __builtin_fmaf(D::hi(yb[k]), o, nz);
  }
}

// max |y| over a chunk of rounded y.
template <class D>
__device__ __forceinline__ float chunk_amax(const uint32_t (&yb)[4]) {
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) a = fmaxf(a, fmaxf(fabsf(D::lo(yb[k])), fabsf(D::hi(yb[k]))));
  return a;
}

// The same max from the fp32 values before their rounding to the
// activation dtype: rounding to nearest is monotone in magnitude, so the
// largest rounded magnitude is the rounding of the largest magnitude.
template <class D>
__device__ __forceinline__ float rounded_amax(const float (&y32)[kVec]) {
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < kVec; ++k) a = fmaxf(a, fabsf(y32[k]));
  return D::lo(D::pack(a, 0.0f));
}

// fl32(a / 6), correctly rounded, for a block amax a >= 0 that a bf16 or
// an fp16 holds (every amax the kernels pass: the max of a block of
// rounded y): the reciprocal r = fl32(1/6), q0 = fl(a r) and one remainder
// correction q0 + (a - 6 q0) r (FMA, one rounding).  For those 60032
// values one correction is exact (checked in exact rational arithmetic by
// tests/test_host_arith.py; for arbitrary fp32 a a second one would be
// needed).  3 VALU instructions instead of the ~10 of an IEEE division.
__device__ __forceinline__ float div6(float a) {
  const float r = 1.0f / kE2M1Max;
  const float q = a * r;
  return __builtin_fmaf(-__builtin_fmaf(q, kE2M1Max, -a), r, q);
}

// NVFP4 block scale: S = E4M3(min(gs * (amax / 6), 448)).
__device__ __forceinline__ uint32_t nvfp4_scale_code(float amax, float gs) {
  const float u = fminf(gs * div6(amax), kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u, 0.0f, __builtin_bit_cast(int, u), false) & 0xffu;
}

// Element multiplier o = gs / decode(S), 0 for a zero scale.
__device__ __forceinline__ float nvfp4_elem_scale(uint32_t s_code, float gs) {
  const float sigma = __builtin_amdgcn_cvt_f32_fp8((int)s_code, 0);
  return sigma == 0.0f ? 0.0f : gs / sigma;
}

// The element multiplier of every E4M3 code a block scale can take (0 ..
// 0x7F), filled once per workgroup into LDS by its threads (visible to all
// after the next barrier): a block then looks o up instead of dividing.
constexpr int kNvfp4Codes = 128;
__device__ __forceinline__ void nvfp4_fill_table(float *tab, float gs, unsigned tid, unsigned nthr) {
  for (unsigned i = tid; i < (unsigned)kNvfp4Codes; i += nthr) tab[i] = nvfp4_elem_scale(i, gs);
}

// rstd = 1 / sqrt(sum(h^2) / H + eps) in fp32 from the row's sum of squares
// and inv_h = 1 / H: a multiply, an add and the hardware reciprocal square
// root (1 ulp), a few fp32 ulps from the exact value like any fp32
// evaluation order, far inside the one unit of the 16-bit output the
// result is rounded to.  Arguments below 2^-100 (eps = 0 and tiny rows) are
// scaled by 2^64 first so the instruction never sees a subnormal.
__device__ __forceinline__ float row_rstd(float sum_sq, float inv_h, float eps) {
  const float v = __builtin_fmaf(sum_sq, inv_h, eps);
  const bool tiny = v < 0x1p-100f;
  const float r = __builtin_amdgcn_rsqf(tiny ? v * 0x1p64f : v);
  return tiny ? r * 0x1p32f : r;
}

// MXFP8 block scale: 2^e with e = floor(log2(amax)) - 8 (8 is the exponent
// of E4M3's largest normal, 448 = 1.75 * 2^8) clamped below at -127, the OCP
// MX scale rule.  The E8M0 code e + 127 is then the biased fp32 exponent of
// amax minus 8, floored at 0 (a zero or subnormal amax gives 0).  amax >= 0;
// the code is at most 247 for any bit pattern.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const uint32_t be = __float_as_uint(amax) >> 23;
  return be > 8u ? be - 8u : 0u;
}

// 2^-e for an E8M0 code <= 247: the fp32 with biased exponent 254 - code
// (a normal number, 2^127 down to 2^-120).  Scaling y by it is exact unless
// the product falls below 2^-126, which encodes to a signed zero either way.
__device__ __forceinline__ float mx_elem_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// Byte offset of block scale (row m, block b) in the 128x4-tiled layout;
// ktiles = round_up(H/16, 4) / 4.  It is the sum of a part that depends on
// the row only (its 128-row tile band, its 16-byte line inside the tile and
// its 4-byte slot in that line) and one that depends on the block only (its
// 512-byte tile along the row and its byte in the slot), so a row loop can
// keep the block part in a register and form the row part in scalars.
__device__ __forceinline__ size_t swz128x4_row(int64_t m, int ktiles) {
  return (size_t)(m >> 7) * (size_t)ktiles * 512u + (size_t)(m & 31) * 16u + (size_t)((m >> 5) & 3) * 4u;
}
__device__ __forceinline__ uint32_t swz128x4_col(int b) { return (uint32_t)(b >> 2) * 512u + (uint32_t)(b & 3); }
__device__ __forceinline__ size_t swz128x4(int64_t m, int b, int ktiles) {
  return swz128x4_row(m, ktiles) + swz128x4_col(b);
}

// Workgroup -> row for NVFP4.  Workgroups are dispatched round-robin over the
// 8 XCDs (workgroup b runs on XCD b % 8).  Inside every full span of 1024
// rows, XCD x takes the whole 128-row tile x, so the 32 rows that share each
// 128-byte line of the 128x4-tiled scales write it through one XCD's L2 and
// the line reaches HBM once (measured: scale writes drop from ~2x to 1x,
// 5% faster at M = 8192).  Rows of a ragged last span map to themselves.
// Inside a tile the rows go in order, except with LINES: then the 32 rows of
// each line group (rows 8 g .. 8 g + 7 and their partners 32, 64 and 96
// rows on) come one after another, so a looping launch that covers half a
// span per pass completes each scale line in one pass (1.3-5% faster for
// rows with a residual at M = 2048 ... 16384, H = 5120, on 512 workgroups;
// 2% slower on 1024, and 8% slower with one workgroup per row, where rows
// in order read memory in order).
template <bool LINES = false>
__device__ __forceinline__ int64_t nvfp4_row_of_block(int64_t b, int64_t M) {
  if ((((b >> 10) + 1) << 10) > M) return b;
  const int64_t lo = b & 1023, i = lo >> 3;
  const int64_t in_tile = LINES ? ((i >> 5) << 3) + (i & 7) + (((i >> 3) & 3) << 5) : i;
  return ((b >> 10) << 10) + ((lo & 7) << 7) + in_tile;
}

// ----------------------------------------------------------------------------
// Cross-lane reductions.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}

// Value of the neighbouring lane (lane ^ 1): DPP quad_perm [1, 0, 3, 2].
__device__ __forceinline__ float dpp_swap_adjacent(float v) { return dpp<0xB1>(v); }

// max of two non-negative floats (block amaxes) as integers: their bit
// patterns order as their values, and the integer max needs none of the
// NaN quieting fmaxf adds under IEEE rules.
__device__ __forceinline__ float max_nonneg(float a, float b) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)));
}

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

// Sum over aligned groups of LPR lanes (LPR a power of two <= 64, all lanes
// active), returned to every lane of the group.
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

// ----------------------------------------------------------------------------
// Gemma (1 + w) or plain (w) RMSNorm scaling of t = h * rstd in IEEE fp32:
// t * fl(1 + w) (two fp32 roundings, then one to the activation dtype: within
// one unit of that dtype of the exact value).  Plain IEEE products also give
// every zero y the sign of h * rstd * (1 + w): fl(1 + w) is +0 for w = -1,
// and t keeps the sign of h.
template <bool GEMMA>
__device__ __forceinline__ float norm_factor(float w) {
  if constexpr (GEMMA) return 1.0f + w;
  return w;
}

template <bool GEMMA>
__device__ __forceinline__ float norm_scale(float t, float w) {
  return t * norm_factor<GEMMA>(w);
}

// Quantize one 8-element chunk of y (yb: four words of two values already
// rounded to the activation dtype D; amax: max |y| over the chunk) of row
// `row`, chunk `ch`, and store its codes (and, for NVFP4, from the even lane
// of the pair, the block scale; for MXFP8, from the first lane of the quad,
// the E8M0 scale).  NVFP4 needs the neighbouring lane to hold the other half
// of the 16-element block and to run this too; MXFP8 likewise needs the
// aligned quad of lanes (4 x 8 = 32 elements) to hold chunks 4k..4k+3 and
// all run it.  TABLE: NVFP4 looks the element multiplier up in otab, the
// workgroup's table (nvfp4_fill_table), instead of dividing.  active =
// false: the lane computes (its DPP partners may need its values) but
// stores nothing.
template <class D, int MODE, bool TABLE = false>
__device__ __forceinline__ void quant_store_chunk(const uint32_t (&yb)[4], float amax, const QuantScale &qs,
                                                  uint8_t *__restrict__ q, uint8_t *__restrict__ bs,
                                                  int64_t row, unsigned ch, int nchunk, int ktiles,
                                                  const float *otab = nullptr, bool active = true) {
  if constexpr (MODE == kModeNvfp4) {
    amax = max_nonneg(amax, dpp_swap_adjacent(amax));
    const uint32_t sc = nvfp4_scale_code(amax, qs.s);
    float o;
    if constexpr (TABLE) o = otab[sc & (kNvfp4Codes - 1)];
    else o = nvfp4_elem_scale(sc, qs.s);
    float v[kVec];
    scale_chunk<D>(yb, o, qs.nz, v);
    const uint32_t codes = e2m1x8(v);
    uint32_t *qrow = reinterpret_cast<uint32_t *>(q + (size_t)row * (size_t)nchunk * 4);
    if (active) __builtin_nontemporal_store(codes, &qrow[ch]);
    if (active && (ch & 1) == 0) (bs + swz128x4_row(row, ktiles))[swz128x4_col((int)(ch >> 1))] = (uint8_t)sc;
  } else if constexpr (MODE == kModeMxfp8) {
    amax = max_nonneg(amax, dpp<0xB1>(amax));   // lane ^ 1
    amax = max_nonneg(amax, dpp<0x4E>(amax));   // lane ^ 2
    const uint32_t sc = mx_scale_code(amax);
    float v[kVec];
    scale_chunk<D>(yb, mx_elem_scale(sc), qs.nz, v);
    const u32x2 packed = {e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7])};
    u32x2 *qrow = reinterpret_cast<u32x2 *>(q + (size_t)row * (size_t)nchunk * 8);
    if (active) __builtin_nontemporal_store(packed, &qrow[ch]);
    if (active && (ch & 3) == 0) bs[(size_t)row * (size_t)(nchunk >> 2) + (ch >> 2)] = (uint8_t)sc;
  } else if constexpr (MODE == kModeFp8) {
    const u32x2 codes = fp8_codes<D>(yb, qs);
    u32x2 *qrow = reinterpret_cast<u32x2 *>(q + (size_t)row * (size_t)nchunk * 8);
    if (active) __builtin_nontemporal_store(codes, &qrow[ch]);
  }
}

// MXFP8 quant of one whole 32-element block held by one thread (the scalar
// kernels): codes to q[0..31] with byte stores (any alignment); returns the
// E8M0 scale code.
__device__ __forceinline__ uint32_t mx_block_store(const float (&yv)[kMxBlock], uint8_t *q) {
  float amax = 0.0f;
  for (int k = 0; k < kMxBlock; ++k) amax = fmaxf(amax, fabsf(yv[k]));
  const uint32_t sc = mx_scale_code(amax);
  const float o = mx_elem_scale(sc);
  for (int k = 0; k < kMxBlock; k += 4) {
    const uint32_t w = e4m3x4(yv[k] * o, yv[k + 1] * o, yv[k + 2] * o, yv[k + 3] * o);
    for (int i = 0; i < 4; ++i) q[k + i] = (uint8_t)(w >> (8 * i));
  }
  return sc;
}

// ----------------------------------------------------------------------------
// Host side.

constexpr int64_t kMaxGrid = ((int64_t)1 << 31) - 1;

struct FusedArgs {
  const void *x;
  void *res;        // nullptr: no residual
  const void *w;
  const float *scale;
  float eps;
  int64_t M;
  int64_t H;
  void *q;
  void *bs;         // NVFP4 128x4-tiled scales, MXFP8 (M, H/32) scales
  void *y;          // nullptr: y not written
  bool gemma;       // (1 + w) if true, w if false
  hipStream_t st;
  void *res_out;    // nullptr: the updated residual goes back into res
};

struct QuantArgs {
  const void *y;
  const float *scale;
  int64_t M;
  int64_t H;
  void *q;
  void *bs;
  hipStream_t st;
};

// One translation unit per (dtype, mode) instantiates the fused kernels.
hipError_t fused_bf16_fp8(const FusedArgs &a);
hipError_t fused_bf16_nvfp4(const FusedArgs &a);
hipError_t fused_bf16_none(const FusedArgs &a);
hipError_t fused_fp16_fp8(const FusedArgs &a);
hipError_t fused_fp16_nvfp4(const FusedArgs &a);
hipError_t fused_fp16_none(const FusedArgs &a);
hipError_t fused_bf16_mxfp8(const FusedArgs &a);
hipError_t fused_fp16_mxfp8(const FusedArgs &a);
hipError_t quant_bf16_fp8(const QuantArgs &a);
hipError_t quant_bf16_nvfp4(const QuantArgs &a);
hipError_t quant_fp16_fp8(const QuantArgs &a);
hipError_t quant_fp16_nvfp4(const QuantArgs &a);
hipError_t quant_bf16_mxfp8(const QuantArgs &a);
hipError_t quant_fp16_mxfp8(const QuantArgs &a);

}  // namespace gnq
