// Fused decode step: the op in static FP8 mode (residual add + Gemma
// RMSNorm + FP8 quant of a few token rows) and its consumer linear (the
// quantized activation times an FP8 weight) in one launch, up to 3 rows.
// From 4 rows on, the step runs the op and the decode GEMM as two launches:
// the one-launch kernel's per-workgroup norm of every row (about 18 VALU
// operations per element) then costs more than the second launch (at
// H = N = 4096: 8.9 against 8.6 us at 4 rows, 11.7 against 8.7 at 8).
//
// The `fused_norm_quant` page launches the op with an early trigger so the
// consumer GEMM's weight fetch overlaps the norm at small batches (its launch
// comment: a ~2% win up to 128 rows).  HIP has no such launch, so here the
// overlap happens inside one kernel, between two kinds of waves of every
// GEMM workgroup:
//   * 4 GEMM waves start the DMA of the workgroup's weight tile (16 weight
//     rows x K bytes, each wave a quarter of K) into LDS, wait for their own
//     quarter, and run the MFMAs over it;
//   * 8 norm waves meanwhile load the activation rows (x, residual: M <= 8
//     rows, from L2 once the first workgroup has pulled them in) and form
//     the rows' add + norm + FP8 codes (every workgroup redundantly) into
//     LDS.
// The split is what lets the two overlap: a wave's vector-memory counter
// covers only its own loads, so a norm wave's wait for its activation rows
// never includes the weight DMA (issued by other waves), whereas one wave
// issuing both would have to wait for the DMA before its first add.
// Workgroup 0's norm waves also store the op's outputs (updated residual,
// codes, and y if asked).  Nothing waits on another workgroup.  Because the
// other workgroups read the residual while workgroup 0 writes, the updated
// residual goes to its own buffer (residual_out), not in place.
//
// Bit-for-bit equal to the two launches it replaces:
//  * the op: the row's sum of squares is formed in exactly the order of the
//    op's kernel for this H (one 8-element chunk per thread of the op's
//    workgroup of H / 8 threads, whose waves the norm waves take over one
//    (row, wave) pair at a time; per-wave DPP sums; the partials added in
//    wave order), and every element goes through the same fp32 operations;
//  * the consumer GEMM: the decode GEMM's K split over 4 waves, its MFMA
//    sequence (32 x 32 x 64 block-scaled FP8 at unit scale, rows clamped to
//    M - 1, weight rows repeated modulo 16) and its fixed-order reduction.
#include "gnq_common.hpp"
#include "gnq_decode.hpp"
#include "gnq_gemm.hpp"
#include "gnq_mfma.hpp"

namespace gnq {
namespace {

constexpr int kFdGemmWaves = 4;     // waves 0..3: weight DMA + MFMAs (K split 4 ways)
constexpr int kFdNormWaves = 8;     // waves 4..11: add + norm + quant of the rows
constexpr int kFdThreads = 64 * (kFdGemmWaves + kFdNormWaves);
constexpr int kFdNT = 16;           // weight rows (output columns) per workgroup
constexpr int kFdRowPad = 16;       // bytes after each activation code row (LDS banks)

// Workgroup barrier for LDS writes only: __syncthreads' release fence would
// also make the GEMM waves wait for their weight DMA still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}

// LDS (static): the weight tile (wave-major: GEMM wave w's K range of all 16
// rows, kq bytes per row, 16-byte chunks XOR-swizzled by row % 8), the
// activation codes (MR rows of K + 16 bytes) and the row partial sums.
__host__ __device__ constexpr int fd_lds_bytes(int K, int MR) {
  return kFdNT * K + MR * (K + kFdRowPad) + MR * 8 * 4;
}

template <class D, int MR, int K, bool HAS_RES, bool WY>
__global__ void __launch_bounds__(kFdThreads)
fused_norm_quant_gemm_decode(const u32x4 *__restrict__ x, const u32x4 *__restrict__ res,
                             u32x4 *__restrict__ res_out, const u32x4 *__restrict__ w,
                             const float *__restrict__ scale_ptr, float eps, int M,
                             const uint8_t *__restrict__ B, const float *__restrict__ b_scale, int N,
                             uint8_t *__restrict__ q, u32x4 *__restrict__ y, uint16_t *__restrict__ C) {
  constexpr int kNchunk = K / kVec;                 // 16-byte chunks of an activation row
  constexpr int kVwaves = kNchunk / kWave;          // the op's waves for this H (2, 4, 8)
  constexpr int kRowsPerPass = kFdNormWaves / kVwaves;            // rows the norm waves cover at once
  constexpr int kUnits = (MR + kRowsPerPass - 1) / kRowsPerPass;  // rows per norm wave
  constexpr int kq = K / kFdGemmWaves;              // a GEMM wave's K range in bytes
  constexpr int kSegs = kFdNT * kq / 1024;          // 1 KB DMA segments per GEMM wave
  constexpr int kAStride = K + kFdRowPad;
  static_assert(kNchunk % kWave == 0 && kFdNormWaves % kVwaves == 0 && kSegs >= 1 && kSegs < 64, "shape");
  // Separate LDS objects, so the compiler can tell the DMA's destination
  // from the LDS the norm uses.
  __shared__ __attribute__((aligned(16))) uint8_t wtile[kFdNT * K];
  __shared__ __attribute__((aligned(16))) uint8_t at[MR * kAStride];
  __shared__ float part[MR * 8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * kFdNT;
  const float s = *scale_ptr;

  if (wave < kFdGemmWaves) {
    // GEMM wave: start the DMA of its K range of the weight tile.
    uint8_t *wt = wtile + wave * kFdNT * kq;
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      // lane l lands at byte 16 l of segment i: weight row o / kq, physical
      // chunk (o % kq) / 16, which holds logical chunk p ^ (row % 8)
      const int o = i * 1024 + lane * 16;
      const int row = o / kq, c = ((o % kq) >> 4) ^ (row & 7);
      const int n = min(n0 + row, N - 1);
      dma16(B + (size_t)n * K + wave * kq + c * 16, wt + i * 1024);
    }
    lds_barrier();   // the rows' partial sums (norm waves)
    lds_barrier();   // the activation codes (norm waves)
  } else {
    // Norm wave: op wave vw of rows m0, m0 + kRowsPerPass, ...
    const int nw = wave - kFdGemmWaves;
    const int vw = nw % kVwaves, m0 = nw / kVwaves;
    const int ch = vw * kWave + lane;               // this lane's 16-byte chunk of a row
    const QuantScale qs = quant_scale(s, true);
    u32x4 xa[kUnits], ra[kUnits];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      const size_t at_ = (size_t)min(m0 + kRowsPerPass * j, M - 1) * kNchunk + ch;
      xa[j] = x[at_];
      if constexpr (HAS_RES) ra[j] = res[at_];
    }
    const u32x4 wa = w[ch];

    // h = RN(x + r), the lane's sum of squares in the op's order, the op
    // wave's DPP sum.
    uint32_t hb[kUnits][4];
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (HAS_RES)
          hb[j][e] = D::pack(D::lo(xa[j][e]) + D::lo(ra[j][e]), D::hi(xa[j][e]) + D::hi(ra[j][e]));
        else
          hb[j][e] = xa[j][e];
        const float a = D::lo(hb[j][e]), b = D::hi(hb[j][e]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(b, b, ss);
      }
      ss = wave_sum(ss);
      const int m = m0 + kRowsPerPass * j;
      if (m < M && lane == 0) part[m * 8 + vw] = ss;
    }
    lds_barrier();

    const float inv_h = __builtin_amdgcn_rcpf((float)(kNchunk * kVec));
    const bool store = blockIdx.x == 0;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      const int m = m0 + kRowsPerPass * j;
      if (m >= M) break;
      float tot = 0.0f;
      for (int i = 0; i < kVwaves; ++i) tot += part[m * 8 + i];
      const float rstd = row_rstd(tot, inv_h, eps);
      uint32_t yb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ta = __builtin_fmaf(D::lo(hb[j][e]), rstd, qs.nz);
        const float tb = __builtin_fmaf(D::hi(hb[j][e]), rstd, qs.nz);
        yb[e] = D::pack(norm_scale<true>(ta, D::lo(wa[e])), norm_scale<true>(tb, D::hi(wa[e])));
      }
      const u32x2 codes = fp8_codes<D>(yb, qs);
      *reinterpret_cast<u32x2 *>(at + m * kAStride + ch * 8) = codes;
      if (store) {
        reinterpret_cast<u32x2 *>(q + (size_t)m * K)[ch] = codes;
        if constexpr (HAS_RES) res_out[(size_t)m * kNchunk + ch] = u32x4{hb[j][0], hb[j][1], hb[j][2], hb[j][3]};
        if constexpr (WY) y[(size_t)m * kNchunk + ch] = u32x4{yb[0], yb[1], yb[2], yb[3]};
      }
    }
    lds_barrier();   // activation codes complete
  }

  // The GEMM waves' K ranges once each wave's own DMA has landed.
  f32x16 acc = f32x16{0};
  if (wave < kFdGemmWaves) {
    wait_vmcnt<0>();
    const int r = lane & 31, h = lane >> 5;
    const int am = min(r, M - 1), bn = r % kFdNT;
    const uint8_t *arow = at + am * kAStride + wave * kq;
    const uint8_t *brow = wtile + wave * kFdNT * kq + bn * kq;
#pragma unroll 4
    for (int t = 0; t < kq / 64; ++t) {
      const int c0 = 4 * t + h, c1 = 4 * t + 2 + h;   // logical 16-byte chunks of the step
      const u32x4 alo = *reinterpret_cast<const u32x4 *>(arow + c0 * 16);
      const u32x4 ahi = *reinterpret_cast<const u32x4 *>(arow + c1 * 16);
      const u32x4 blo = *reinterpret_cast<const u32x4 *>(brow + ((c0 ^ (bn & 7)) << 4));
      const u32x4 bhi = *reinterpret_cast<const u32x4 *>(brow + ((c1 ^ (bn & 7)) << 4));
      const i32x8 af = {(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
      const i32x8 bf = {(int)blo[0], (int)blo[1], (int)blo[2], (int)blo[3], (int)bhi[0], (int)bhi[1], (int)bhi[2], (int)bhi[3]};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc, 0, 0, 0, 127, 0, 127);
    }
  }

  // The GEMM waves' partial tiles summed in wave order over the (idle)
  // weight tile's LDS.
  __syncthreads();
  float *red = reinterpret_cast<float *>(wtile);
  if (wave < kFdGemmWaves) {
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave * 1024 + v * 64 + lane] = acc[v];
  }
  __syncthreads();
  const float sc = s * (*b_scale);
  for (int e = tid; e < 1024; e += kFdThreads) {
    const int v = (e >> 6) & 15, l = e & 63;
    const int tr = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    const int tc = l & 31;
    const int col = n0 + tc;
    if (tr < M && tc < kFdNT && col < N) {
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kFdGemmWaves; ++ww) sum += red[ww * 1024 + e];
      C[(size_t)tr * (size_t)N + col] = (uint16_t)(Bf16::pack(sum * sc, 0.0f) & 0xffffu);
    }
  }
}

template <class D, int MR, int K, bool HAS_RES, bool WY>
hipError_t launch_fd(const FusedDecodeArgs &a) {
  // all of the kernel's LDS is static (its three arrays)
  static_assert(fd_lds_bytes(K, MR) <= 160 * 1024, "LDS");
  const dim3 grid((unsigned)((a.N + kFdNT - 1) / kFdNT));
  return launch(fused_norm_quant_gemm_decode<D, MR, K, HAS_RES, WY>, grid, dim3(kFdThreads), 0, a.st,
                (const u32x4 *)a.x, (const u32x4 *)a.res, (u32x4 *)a.res_out, (const u32x4 *)a.w, a.scale,
                a.eps, (int)a.M, (const uint8_t *)a.b, a.b_scale, (int)a.N, (uint8_t *)a.q, (u32x4 *)a.y,
                (uint16_t *)a.out);
}

template <class D, int MR, int K>
hipError_t fd_res_y(const FusedDecodeArgs &a) {
  const bool res = a.res != nullptr, wy = a.y != nullptr;
  if (res) return wy ? launch_fd<D, MR, K, true, true>(a) : launch_fd<D, MR, K, true, false>(a);
  return wy ? launch_fd<D, MR, K, false, true>(a) : launch_fd<D, MR, K, false, false>(a);
}

template <class D, int MR>
hipError_t fd_k(const FusedDecodeArgs &a) {
  switch (a.H) {
    case 1024: return fd_res_y<D, MR, 1024>(a);
    case 2048: return fd_res_y<D, MR, 2048>(a);
    default: return fd_res_y<D, MR, 4096>(a);
  }
}

template <class D>
hipError_t fd_rows(const FusedDecodeArgs &a) {
  if (a.M <= 1) return fd_k<D, 1>(a);
  if (a.M <= 2) return fd_k<D, 2>(a);
  return fd_k<D, 4>(a);
}

// From 4 rows on, the two launches: the op (its updated residual written to
// residual_out) and the decode GEMM, the same kernels the two separate calls
// run.
hipError_t two_launches(const FusedDecodeArgs &a, bool bf16) {
  FusedArgs op{a.x,  const_cast<void *>(a.res), a.w, a.scale, a.eps, a.M, a.H, a.q, nullptr, a.y,
               true, a.st, a.res ? a.res_out : nullptr};
  const hipError_t e = bf16 ? fused_bf16_fp8(op) : fused_fp16_fp8(op);
  if (e != hipSuccess) return e;
  return gemm_fp8(false, a.q, nullptr, a.b, nullptr, a.scale, a.b_scale, a.M, a.N, a.H, a.out, a.st);
}

}  // namespace

bool fused_decode_supported(int64_t M, int64_t H) {
  return M >= 1 && M <= kFusedDecodeMaxRows && (H == 1024 || H == 2048 || H == 4096);
}

hipError_t fused_decode(const FusedDecodeArgs &a, bool bf16) {
  if (a.M > kFusedDecodeOneLaunchRows) return two_launches(a, bf16);
  return bf16 ? fd_rows<Bf16>(a) : fd_rows<Fp16>(a);
}

}  // namespace gnq
