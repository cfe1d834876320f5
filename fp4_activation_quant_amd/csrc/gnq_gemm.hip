// Consumer GEMM of the quantized activation: C[M, N] = dq(A) * dq(B)^T in
// bf16, A the (M, K) activation codes the op wrote and B the (N, K) weight
// codes in the same format, both K-contiguous (the pre-quantized input path
// of the quantized linears on the PR conversation page).  Three formats:
//  * MXFP8: E4M3 codes with row-major E8M0 scales (rows, K / 32), fed to the
//    gfx950 block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) as they are;
//  * static FP8: E4M3 codes with one fp32 scale per tensor: the same MFMA at
//    unit block scale, the product of the two tensor scales applied to the
//    fp32 accumulator;
//  * NVFP4: packed E2M1 codes with 128x4-tiled E4M3 block scales, dequantized
//    exactly to fp16 in registers for the fp16 MFMA (gemm_nvfp4 below).
//
// Operand layout of the MFMA (32 x 32 output, K = 64 per instruction,
// measured on the chip with a one-wave probe): lane l supplies row (or
// column) l % 32; its 32 bytes are two 16-byte halves, bytes 0..15 from the
// first 32-element K block and bytes 16..31 from the second, lanes 0..31
// holding the low 16 elements of each block and lanes 32..63 the high 16.
// The scale operand of lane l is the E8M0 code of (row l % 32, block l / 32).
// Accumulator register v of lane l is C[8 * (v / 4) + 4 * (l / 32) + v % 4]
// [l % 32].
//
// Kernels (the dispatchers gemm_fp8 and gemm_nvfp4 at the end pick one by
// shape and workgroup count):
//  * gemm_fp8_tn_dma<.., T>: FP8 / MXFP8 for K % 512 == 0 on T x T
//    workgroup tiles (T = 256: 8 waves of 64 x 128, two per SIMD, measured
//    ~9% faster at 8192 x 4096 x 4096 than 4 waves of 128 x 128; T = 128:
//    4 waves of 64 x 64), K advancing 64 bytes per step
//    through LDS stages filled by direct global->LDS DMA three steps ahead,
//    fragment reads pipelined one step ahead of the MFMAs;
//  * gemm_fp8_tn: the register-staged two-stage kernel on 256 x 256 tiles
//    for other K;
//  * gemm_fp8_decode, gemm_fp8_skinny: up to 256 rows, small tiles whose
//    waves split K (the weight stream is the cost);
//  * gemm_nvfp4_gemv (a few rows, narrow weight), gemm_nvfp4_k (32- to 128-row tiles,
//    waves splitting K) and gemm_nvfp4_big (256 x 256): NVFP4.
// LDS rows of 64 bytes have their 16-byte chunks XOR-swizzled by row to
// spread LDS banks.  Rows beyond M or N are clamped on load and masked on
// store; a K tail of 32 (K % 64 == 32) loads zeros for the missing block.
#include <atomic>

#include "gnq_common.hpp"
#include "gnq_gemm.hpp"
#include "gnq_mfma.hpp"

namespace gnq {

constexpr int kGemmThreads = 256;
constexpr int kGemmTile = 256;                // output rows and columns per workgroup
constexpr int kGemmWaveTile = 128;            // per wave
constexpr int kGemmK = 64;                    // K bytes per step
constexpr int kGemmOperandBytes = kGemmTile * kGemmK;     // 16 KB per operand per stage

// Chunk swizzle of a 64-byte LDS row: chunk c of row r sits at position
// c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) % 4.  The 16-byte reads of 8 and of
// 16 consecutive rows at one chunk then cover 128 and 256 distinct bytes
// modulo 256 (no bank conflict with 32 or 64 four-byte banks; the plain
// ((r >> 1) % 4) swizzle left a 2-way conflict, measured as 44% of LDS
// cycles).
__device__ __forceinline__ int gemm_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__device__ __forceinline__ int gemm_lds_off(int row, int chunk) {
  return row * kGemmK + ((chunk ^ gemm_swz(row)) << 4);
}

// Output tile of workgroup b.  Workgroups are dealt to the 8 XCDs (each
// with its own L2) round-robin, b % 8; when the tile count is a multiple of
// 8 the tiles are renumbered so that XCD x works through the contiguous
// range of tiles x T / 8 .. (x + 1) T / 8 - 1.  In that order tiles go in
// groups of 4 tile rows, column by column, so the ~32 workgroups an XCD
// holds at once cover 4 row tiles of A and 8 column tiles of B: 12 operand
// tiles shared in its L2 instead of 18 (2 x 16) with plain groups of 16 rows
// (measured ~4% faster at 32768 x 8192 x 8192).
constexpr int kGemmGroupRows = 4;
constexpr int kXcds = 8;

__device__ __forceinline__ void gemm_tile_of_block(int b, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int tiles = tiles_m * tiles_n;
  if (tiles % kXcds == 0) b = (b % kXcds) * (tiles / kXcds) + b / kXcds;
  const int per_group = kGemmGroupRows * tiles_n;
  const int first = (b / per_group) * kGemmGroupRows;
  const int rows = min(tiles_m - first, kGemmGroupRows);
  const int p = b % per_group;
  tm = first + p % rows;
  tn = p / rows;
}

__device__ __forceinline__ i32x8 gemm_frag(const uint8_t *base, int row, int h) {
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + gemm_lds_off(row, h));
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + gemm_lds_off(row, 2 + h));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool MX>
__global__ void __launch_bounds__(kGemmThreads)
gemm_fp8_tn(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
            const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
            const float *__restrict__ a_scale, const float *__restrict__ b_scale, int M, int N, int K,
            uint16_t *__restrict__ C, int tiles_m, int tiles, int unit_scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kGemmOperandBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  int tm, tn;
  gemm_tile_of_block(blockIdx.x, tiles_m, tiles / tiles_m, tm, tn);
  const int m0 = tm * kGemmTile, n0 = tn * kGemmTile;
  const int wm = (wave >> 1) * kGemmWaveTile, wn = (wave & 1) * kGemmWaveTile;
  const int ksteps = (K + kGemmK - 1) / kGemmK;
  const int kblocks = K / 32;

  // Global -> LDS staging: each thread moves 16-byte chunk c = tid % 4 of
  // rows tid / 4 + 64 j (j = 0..3) of both operand tiles.
  const int c = tid & 3;
  const uint8_t *a_src[4], *b_src[4];
  int st_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (tid >> 2) + 64 * j;
    const int ar = min(m0 + row, M - 1), br = min(n0 + row, N - 1);
    a_src[j] = A + (size_t)ar * (size_t)K + c * 16;
    b_src[j] = B + (size_t)br * (size_t)K + c * 16;
    st_off[j] = gemm_lds_off(row, c);
  }
  // Scale rows of this lane's four A and four B MFMA tiles.
  size_t sa_row[4], sb_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa_row[i] = (size_t)min(m0 + wm + 32 * i + r, M - 1) * (size_t)kblocks;
    sb_row[i] = (size_t)min(n0 + wn + 32 * i + r, N - 1) * (size_t)kblocks;
  }

  u32x4 a_st[4], b_st[4];
  int sa_cur[4], sb_cur[4], sa_nxt[4], sb_nxt[4];
  auto gload = [&](int ks) {
    const int kb = ks * kGemmK;
    const bool in = kb + c * 16 < K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a_st[j] = in ? *reinterpret_cast<const u32x4 *>(a_src[j] + kb) : u32x4{0, 0, 0, 0};
      b_st[j] = in ? *reinterpret_cast<const u32x4 *>(b_src[j] + kb) : u32x4{0, 0, 0, 0};
    }
  };
  auto sload = [&](int ks, int (&sa)[4], int (&sb)[4]) {
    const int blk = 2 * ks + h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (MX && blk < kblocks) {
        sa[i] = SA[sa_row[i] + blk];
        sb[i] = SB[sb_row[i] + blk];
      } else {
        sa[i] = unit_scale;
        sb[i] = unit_scale;
      }
    }
  };
  auto stage_store = [&](int s) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4 *>(&lds[s][st_off[j]]) = a_st[j];
      *reinterpret_cast<u32x4 *>(&lds[s][kGemmOperandBytes + st_off[j]]) = b_st[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};

  gload(0);
  sload(0, sa_cur, sb_cur);
  stage_store(0);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < ksteps;
    if (more) {
      gload(ks + 1);
      sload(ks + 1, sa_nxt, sb_nxt);
    }
    const uint8_t *a_lds = lds[cur];
    const uint8_t *b_lds = lds[cur] + kGemmOperandBytes;
    i32x8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = gemm_frag(b_lds, wn + 32 * j + r, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x8 af = gemm_frag(a_lds, wm + 32 * i + r, h);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0,
                                                                    sa_cur[i], 0, sb_cur[j]);
    }
    if (more) {
      stage_store(cur ^ 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_cur[i] = sa_nxt[i];
        sb_cur[i] = sb_nxt[i];
      }
    }
    __syncthreads();
  }

  const float s = MX ? 1.0f : (*a_scale) * (*b_scale);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M && col < N)
          C[(size_t)row * (size_t)N + col] = (uint16_t)(Bf16::pack(acc[i][j][v] * s, 0.0f) & 0xffffu);
      }
    }
}

// Direct-to-LDS pipeline (K % 512 == 0): global_load_lds_dwordx4 moves each
// wave's 1 KB segments straight into LDS (lane l fills bytes 16 l .. 16 l +
// 15 of the segment, so lane l fetches the global chunk that the swizzled
// layout puts there), with no register staging, into kGemmStages stages.
// For MXFP8 the E8M0 codes arrive in windows of 8 steps: one 16-byte DMA per
// row (blocks 16 j .. 16 j + 15 of the row) into one of two LDS windows,
// issued a window ahead, so a row's scale line is fetched once per 8 steps
// instead of once per step (4-byte loads from 64 rows per instruction cost
// ~20% when issued every step).  One barrier per step.
constexpr int kGemmStages = 4;
constexpr int kGemmScaleSteps = 8;                                   // K steps per scale window
// LDS layout for a T x T workgroup tile: kGemmStages stages of both
// operands' T rows x kGemmK bytes, then two scale windows of T rows x 16
// bytes per operand (T = 256: 128 KB + 16 KB; T = 128: 64 KB + 8 KB).
__host__ __device__ constexpr int dma_operand_bytes(int T) { return T * kGemmK; }
__host__ __device__ constexpr int dma_stage_bytes(int T) { return 2 * dma_operand_bytes(T); }
__host__ __device__ constexpr int dma_scale_win(int T) { return T * 2 * kGemmScaleSteps; }
__host__ __device__ constexpr int dma_scale_off(int T) { return kGemmStages * dma_stage_bytes(T); }
__host__ __device__ constexpr int dma_lds_bytes(int T) { return dma_scale_off(T) + 2 * 2 * dma_scale_win(T); }

// NW waves per workgroup, each owning TM x TN MFMA tiles (32 x 32) of the
// T x T workgroup tile; the T / 8 one-KB data segments (16 rows each, T / 16
// per operand) and T / 32 scale segments (64 rows each) of a step are split
// evenly over the waves.  The LDS reads are pipelined
// across steps: the fragments and scale codes of step k + 1 are read into a
// second register set while the MFMAs of step k run, so after the barrier a
// wave goes straight to its MFMAs.  The barrier of step k certifies that
// step k + 1's DMA has landed (each wave waits for its own segments first)
// and that every wave has consumed the reads of step k - 1, whose stage the
// DMA issued after it refills (two steps of DMA ahead of the reads).
template <bool MX, int NW, int TM, int TN, int T>
__global__ void __launch_bounds__(64 * NW)
gemm_fp8_tn_dma(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                const float *__restrict__ a_scale, const float *__restrict__ b_scale, int M, int N,
                int K, uint16_t *__restrict__ C, int tiles_m, int tiles, int unit_scale) {
  static_assert(T == 128 || T == 256, "workgroup tile");
  static_assert((T / 32 / TM) * (T / 32 / TN) == NW, "waves must tile the T x T workgroup tile");
  static_assert(kGemmStages == 4, "the waits below assume four stages");
  static_assert((T / 8) % NW == 0 && (T / 32) % NW == 0, "segments split evenly over the waves");
  constexpr int kSegs = T / 8 / NW;
  constexpr int kScaleSegs = T / 32 / NW;
  constexpr int kWavesN = T / 32 / TN;
  constexpr int kOperandBytes = dma_operand_bytes(T), kStageBytes = dma_stage_bytes(T);
  constexpr int kScaleWin = dma_scale_win(T), kScaleOff = dma_scale_off(T);
  constexpr int kMfma = TM * TN, kUnits = TM + TN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  int tm, tn;
  gemm_tile_of_block(blockIdx.x, tiles_m, tiles / tiles_m, tm, tn);
  const int m0 = tm * T, n0 = tn * T;
  const int wm = (wave / kWavesN) * 32 * TM, wn = (wave % kWavesN) * 32 * TN;
  const int ksteps = K / kGemmK;
  const int kblocks = K / 32;

  const bool fetch_b = kSegs * wave >= T / 16;
  const uint8_t *src = fetch_b ? B : A;
  const int lim = fetch_b ? N - 1 : M - 1, base_row = fetch_b ? n0 : m0;
  const int seg0 = (kSegs * wave) % (T / 16);
  const uint8_t *seg_src[kSegs];
#pragma unroll
  for (int j = 0; j < kSegs; ++j) {
    const int row = 16 * (seg0 + j) + (lane >> 2);
    const int chunk = (lane & 3) ^ gemm_swz(row);
    seg_src[j] = src + (size_t)min(base_row + row, lim) * (size_t)K + chunk * 16;
  }
  const bool sfetch_b = kScaleSegs * wave >= T / 64;
  const int sseg0 = (kScaleSegs * wave) % (T / 64);
  const uint8_t *sc_src[kScaleSegs];
#pragma unroll
  for (int t = 0; t < kScaleSegs; ++t) {
    const int lim_s = sfetch_b ? N - 1 : M - 1, base_s = sfetch_b ? n0 : m0;
    sc_src[t] = MX ? (sfetch_b ? SB : SA) + (size_t)min(base_s + 64 * (sseg0 + t) + lane, lim_s) * (size_t)kblocks
                   : nullptr;
  }
  // DMA of step `from` into the stage of step ks (from != ks only for the
  // refetches past the last step), and of scale window `from` into the
  // buffer of window w.
  auto issue_seg = [&](int ks, int from, int j) {
    uint8_t *dst = smem + (ks % kGemmStages) * kStageBytes + (fetch_b ? kOperandBytes : 0) + seg0 * 1024;
    dma16(seg_src[j] + from * kGemmK, dst + j * 1024);
  };
  auto issue = [&](int ks, int from) {
#pragma unroll
    for (int j = 0; j < kSegs; ++j) issue_seg(ks, from, j);
  };
  auto issue_scales = [&](int w, int from) {
    uint8_t *sdst = smem + kScaleOff + (w & 1) * 2 * kScaleWin + (sfetch_b ? kScaleWin : 0) +
                    sseg0 * 1024;
#pragma unroll
    for (int t = 0; t < kScaleSegs; ++t) dma16(sc_src[t] + 16 * from, sdst + t * 1024);
  };
  const int chunks = ksteps / 8;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{0};
  i32x8 af[2][TM], bf[2][TN];
  // MXFP8: this lane's E8M0 codes of the current 8-step scale window, for
  // each operand unit (B tiles, then A tiles): the byte of step j at byte
  // j % 4 of word j / 4.  Loaded once per window by a 16-byte LDS read per
  // unit (16-byte rows: no bank conflicts; per-step byte reads of 32 rows
  // 16 bytes apart conflicted two-way) and packed to this lane's half.
  uint32_t swin[kUnits][2];
  // LDS byte offsets of this lane's fragment rows, one per (stage pair,
  // operand, 16-byte half).  The swizzle of rows wm + 32 i + r depends on r
  // only, so tile, stage-in-pair and slot constants become immediate offsets
  // of the reads; the offsets are hidden from the optimizer, which otherwise
  // folds every constant into its own address register (one per read of the
  // unrolled steps) and spills.
  const int swz = gemm_swz(r);
  uint32_t fbase[2][2][2];
#pragma unroll
  for (int sp = 0; sp < 2; ++sp)
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        fbase[sp][op][hh] = (uint32_t)(sp * 2 * kStageBytes + op * kOperandBytes +
                                       ((op ? wn : wm) + r) * kGemmK + (((2 * hh + h) ^ swz) << 4));
        asm volatile("" : "+v"(fbase[sp][op][hh]));
      }
  uint32_t sbase[2];
#pragma unroll
  for (int op = 0; op < 2; ++op) {
    sbase[op] = (uint32_t)(kScaleOff + op * kScaleWin + ((op ? wn : wm) + r) * 16);
    asm volatile("" : "+v"(sbase[op]));
  }
  // bytes h, h + 2, h + 4, h + 6 of a pair of window words (steps 0..3 or
  // 4..7 of this lane's half: lanes 32..63 take the odd blocks)
  const uint32_t sel = 0x06040200u + 0x01010101u * (uint32_t)h;
  auto load_window = [&](uint32_t wofs) {
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int op = u < TN ? 1 : 0, t = u < TN ? u : u - TN;
      const u32x4 w4 = *reinterpret_cast<const u32x4 *>(smem + sbase[op] + wofs + t * 32 * 16);
      swin[u][0] = __builtin_amdgcn_perm(w4[1], w4[0], sel);
      swin[u][1] = __builtin_amdgcn_perm(w4[3], w4[2], sel);
    }
  };
  // the E8M0 code of unit u for step j (0..7) of the window
  auto code_of = [&](int u, int j) -> int {
    return (int)__builtin_amdgcn_ubfe(swin[u][j >> 2], 8 * (j & 3), 8);
  };
  // Read unit u of step ks into register set p: B tile u for u < TN, else
  // A tile u - TN.
  auto read_unit = [&](int ks, int p, int u) {
    const int stg = ks % kGemmStages;
    const int op = u < TN ? 1 : 0, t = u < TN ? u : u - TN;
    const uint32_t imm = (uint32_t)((stg & 1) * kStageBytes + t * 32 * kGemmK);
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(smem + fbase[stg >> 1][op][0] + imm);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(smem + fbase[stg >> 1][op][1] + imm);
    const i32x8 f = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    if (op) bf[p][t] = f;
    else af[p][t] = f;
  };

  // One K step: MFMAs of step ks from register set ks % 2, interleaved with
  // the reads of step ks + 1 into the other set.  The body has no branch (a
  // branch let the compiler sink the MFMAs below later steps' reads): the
  // last steps' DMA refetches the final step into stages no step reads
  // again, and the last step's reads fetch a stale stage and scale slot
  // (inside LDS) that nothing uses.
  auto step = [&](int ks, int u8, int c) {
    const int p = u8 & 1;
    // step ks + 1's segments of this wave: at most step ks + 2's (and a
    // scale window issued after them) may still be in flight
    wait_vmcnt<kSegs>();
    asm volatile("s_barrier" ::: "memory");
    // this step's scale codes, before the last step of a window loads the
    // next window's (the barrier above certifies its DMA has landed)
    int sa[TM], sb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = MX ? code_of(j, u8) : unit_scale;
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = MX ? code_of(TN + i, u8) : unit_scale;
    if (MX && u8 == kGemmScaleSteps - 1)
      load_window((uint32_t)(((c + 1) & 1) * 2 * kScaleWin));
    const int nk = ks + kGemmStages - 1, from = min(nk, ksteps - 1);
    // The DMA of step ks + 3 (each instruction holds the wave for many
    // cycles) and the reads of step ks + 1 are spread between the MFMAs
    // so that one is always queued.
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      const int i = q / TN, j = q % TN;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[p][i], bf[p][j], acc[i][j], 0, 0, 0,
                                                                  sa[i], 0, sb[j]);
      __builtin_amdgcn_sched_barrier(0);
      // unit u of the next step is read after MFMA u * kMfma / kUnits,
      // DMA segment g after MFMA g * kMfma / kSegs + kMfma / (2 kSegs)
#pragma unroll
      for (int u = 0; u < kUnits; ++u)
        if ((u * kMfma) / kUnits == q) read_unit(ks + 1, p ^ 1, u);
#pragma unroll
      for (int g = 0; g < kSegs; ++g)
        if ((g * kMfma) / kSegs + kMfma / (2 * kSegs) == q) issue_seg(nk, from, g);
      if (MX && u8 == 0 && q == kMfma - 1) issue_scales(c + 1, min(c + 1, chunks - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ksteps % 8 == 0 (K % 512 == 0): steps run in chunks of 8, so stage,
  // register set and scale slot are compile-time per step.
  if (MX) issue_scales(0, 0);
#pragma unroll
  for (int p = 0; p < kGemmStages - 1; ++p) issue(p, p);
  wait_vmcnt<kSegs * (kGemmStages - 2)>();
  asm volatile("s_barrier" ::: "memory");
  if (MX) load_window(0);
#pragma unroll
  for (int u = 0; u < kUnits; ++u) read_unit(0, 0, u);
  for (int c = 0; c < chunks; ++c) {
#pragma unroll
    for (int u8 = 0; u8 < 8; ++u8) step(8 * c + u8, u8, c);
  }
  wait_vmcnt<0>();   // the refetches land before the workgroup's LDS is released

  const float s = MX ? 1.0f : (*a_scale) * (*b_scale);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M && col < N)
          // streamed out (non-temporal): 3-5% faster at 8192 x 4096 x 4096, the
          // same at 32768 x 8192 x 8192
          __builtin_nontemporal_store((uint16_t)(Bf16::pack(acc[i][j][v] * s, 0.0f) & 0xffffu),
                                      &C[(size_t)row * (size_t)N + col]);
      }
    }
}

// Explicit instantiations: the kernels are referenced only from the launch
// template below, and without these the device stubs were not emitted.
#define GNQ_GEMM_DMA_INST(MX, NW, TM, TN, T)                                                     \
  template __global__ void gemm_fp8_tn_dma<MX, NW, TM, TN, T>(                                   \
      const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *, const float *,         \
      const float *, int, int, int, uint16_t *, int, int, int);
GNQ_GEMM_DMA_INST(true, 8, 2, 4, 256)
GNQ_GEMM_DMA_INST(false, 8, 2, 4, 256)
GNQ_GEMM_DMA_INST(true, 4, 2, 2, 128)
GNQ_GEMM_DMA_INST(false, 4, 2, 2, 128)
#undef GNQ_GEMM_DMA_INST

template <bool MX, int NW, int TM, int TN, int T>
hipError_t launch_dma(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                      const float *a_scale, const float *b_scale, int M, int N, int K, uint16_t *C,
                      hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  constexpr int lds = dma_lds_bytes(T);
  const hipError_t e = allow_dynamic_lds((const void *)gemm_fp8_tn_dma<MX, NW, TM, TN, T>, lds, lds_set);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + T - 1) / T, tiles = tiles_m * ((N + T - 1) / T);
  return launch(gemm_fp8_tn_dma<MX, NW, TM, TN, T>, dim3(tiles), dim3(64 * NW), lds, st, A, SA, B, SB,
                a_scale, b_scale, M, N, K, C, tiles_m, tiles, 127);
}


// Skinny GEMM for few activation rows (decode batches, M <= 64 per chunk):
// the weight stream is the whole cost, so each workgroup owns 32 weight rows
// (output columns) and one 64-row chunk of the activation, and its 8 waves
// split K (wave w takes K steps w, w + 8, ...), loading their fragments
// straight from global memory (the activation chunk stays in L2), kSkinnyUnroll
// steps in flight per wave.  The 8 partial 64 x 32 fp32 tiles are summed
// through LDS in a fixed order (deterministic), then rounded to bf16.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyUnroll = 4;
constexpr int kSkinnyRows = 64;                                      // activation rows per chunk
constexpr int kSkinnyLds = kSkinnyWaves * 2 * 16 * 64 * 4;           // 64 KB of partials

__device__ __forceinline__ i32x8 gemm_gfrag(const uint8_t *row_k) {
  // lane's 32 bytes of one 64-byte K step: 16 at +16h and 16 at +32+16h
  // (row_k already includes the +16h)
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(row_k);
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(row_k + 32);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool MX>
__global__ void __launch_bounds__(64 * kSkinnyWaves)
gemm_fp8_skinny(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                const float *__restrict__ a_scale, const float *__restrict__ b_scale, int M, int N, int K,
                uint16_t *__restrict__ C, int unit_scale) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float *part = reinterpret_cast<float *>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * 32, m0 = blockIdx.y * kSkinnyRows;
  const int ksteps = K / kGemmK, kblocks = K / 32;
  const uint8_t *b_row = B + (size_t)min(n0 + r, N - 1) * (size_t)K + 16 * h;
  const uint8_t *a_row0 = A + (size_t)min(m0 + r, M - 1) * (size_t)K + 16 * h;
  const uint8_t *a_row1 = A + (size_t)min(m0 + 32 + r, M - 1) * (size_t)K + 16 * h;
  const uint8_t *sb_row = MX ? SB + (size_t)min(n0 + r, N - 1) * (size_t)kblocks + h : nullptr;
  const uint8_t *sa_row0 = MX ? SA + (size_t)min(m0 + r, M - 1) * (size_t)kblocks + h : nullptr;
  const uint8_t *sa_row1 = MX ? SA + (size_t)min(m0 + 32 + r, M - 1) * (size_t)kblocks + h : nullptr;
  const bool two = m0 + 32 < M;                    // second 32-row tile has rows

  f32x16 acc0 = f32x16{0}, acc1 = f32x16{0};
  for (int ks0 = wave; ks0 < ksteps; ks0 += kSkinnyUnroll * kSkinnyWaves) {
    i32x8 bf[kSkinnyUnroll], af0[kSkinnyUnroll], af1[kSkinnyUnroll];
    int sb[kSkinnyUnroll], sa0[kSkinnyUnroll], sa1[kSkinnyUnroll];
    // all loads of the unrolled steps first (steps past the end load step
    // ks0 again and are not used)
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      const int ks = ks0 + u * kSkinnyWaves < ksteps ? ks0 + u * kSkinnyWaves : ks0;
      const size_t kb = (size_t)ks * kGemmK;
      bf[u] = gemm_gfrag(b_row + kb);
      af0[u] = gemm_gfrag(a_row0 + kb);
      af1[u] = two ? gemm_gfrag(a_row1 + kb) : i32x8{0};
      sb[u] = MX ? (int)sb_row[2 * ks] : unit_scale;
      sa0[u] = MX ? (int)sa_row0[2 * ks] : unit_scale;
      sa1[u] = MX ? (int)sa_row1[2 * ks] : unit_scale;
    }
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      if (ks0 + u * kSkinnyWaves < ksteps) {
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af0[u], bf[u], acc0, 0, 0, 0, sa0[u], 0, sb[u]);
        if (two)
          acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af1[u], bf[u], acc1, 0, 0, 0, sa1[u], 0, sb[u]);
      }
    }
  }
  // partials: part[((wave * 2 + tile) * 16 + v) * 64 + lane]
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    part[((wave * 2 + 0) * 16 + v) * 64 + lane] = acc0[v];
    part[((wave * 2 + 1) * 16 + v) * 64 + lane] = acc1[v];
  }
  __syncthreads();
  const float s = MX ? 1.0f : (*a_scale) * (*b_scale);
  for (int e = tid; e < 2 * 16 * 64; e += 64 * kSkinnyWaves) {
    float sum = 0.0f;
    for (int w = 0; w < kSkinnyWaves; ++w) sum += part[w * 2 * 16 * 64 + e];
    const int tile = e / (16 * 64), v = (e / 64) % 16, l = e % 64;
    const int row = m0 + 32 * tile + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    const int col = n0 + (l & 31);
    if (row < M && col < N)
      C[(size_t)row * (size_t)N + col] = (uint16_t)(Bf16::pack(sum * s, 0.0f) & 0xffffu);
  }
}

template __global__ void gemm_fp8_skinny<true>(const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *,
                                               const float *, const float *, int, int, int, uint16_t *, int);
template __global__ void gemm_fp8_skinny<false>(const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *,
                                                const float *, const float *, int, int, int, uint16_t *, int);

template <bool MX>
hipError_t launch_skinny(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                         const float *a_scale, const float *b_scale, int M, int N, int K, uint16_t *C,
                         hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = allow_dynamic_lds((const void *)gemm_fp8_skinny<MX>, kSkinnyLds, lds_set);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + 31) / 32), (unsigned)((M + kSkinnyRows - 1) / kSkinnyRows));
  return launch(gemm_fp8_skinny<MX>, grid, dim3(64 * kSkinnyWaves), kSkinnyLds, st, A, SA, B, SB,
                a_scale, b_scale, M, N, K, C, 127);
}

// Decode-size GEMM (few activation rows, K % 2048 == 0, K <= 16384): a
// workgroup owns an MT x NT output tile (MT activation rows, NT weight rows)
// and its NW waves split K into contiguous ranges.  Each wave streams its
// range through a private ring of S LDS stages of 128 K-bytes (two MFMA
// steps) by global_load_lds_dwordx4, eight lanes per 128-byte line, so one
// instruction touches 8 cache lines; loading MFMA fragments straight from
// global memory (lane l -> row l % 32) touches 32 lines per instruction and
// left the skinny kernel bound by the address unit at ~16 GB/s per
// workgroup.  A wave needs no barrier: it waits only for its own DMA.  The
// E8M0 codes of the wave's range (K / 32 / NW bytes per row) arrive by
// 16-byte DMA before the data.  A tile narrower than the 32 x 32 MFMA
// repeats its rows in the unused lanes (rows r % MT, r % NT), whose outputs
// are dropped: narrow tiles give more workgroups for few rows, wide ones
// fewer re-reads of both operands.  The NW partial tiles are summed through
// LDS in a fixed order.
constexpr int kDecStepK = 128;                                 // K bytes per stage (two MFMA steps)
constexpr int kDecMaxK = 16384;
constexpr int kDecDataBytes = 128 * 1024;                      // stage rings of the waves
constexpr int kDecLdsMax = 160 * 1024;

// scale rows (weight then activation) per 16-byte piece: 64 per DMA part
__host__ __device__ constexpr int dec_scale_parts(int MT, int NT) { return (MT + NT + 63) / 64; }
// 16-byte pieces per row per wave: K / NW / 512; one KB per part per piece
__host__ __device__ constexpr int dec_lds_bytes(int K, int MT, int NT) {
  return kDecDataBytes + 2 * K * dec_scale_parts(MT, NT);
}

// Chunk swizzle of a 128-byte LDS row: chunk c of row r at slot c ^ g(r),
// g(r) = (r / 2) % 8, so 16-byte reads of 16 consecutive rows at one chunk
// hit 16 distinct slots modulo 256 bytes.
__device__ __forceinline__ int dec_swz(int row) { return (row >> 1) & 7; }

// Wait until at most `out` stages of PER loads each are in flight.
template <int PER, int MAXO>
__device__ __forceinline__ void dec_wait(int out) {
  if constexpr (MAXO == 0) {
    wait_vmcnt<0>();
  } else {
    if (out >= MAXO) wait_vmcnt<PER * MAXO>();
    else dec_wait<PER, MAXO - 1>(out);
  }
}

template <bool MX, int NW, int MT, int NT, int S>
__global__ void __launch_bounds__(64 * NW)
gemm_fp8_decode(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                const float *__restrict__ a_scale, const float *__restrict__ b_scale, int M, int N, int K,
                uint16_t *__restrict__ C, int unit_scale) {
  constexpr int kBSeg = NT / 8, kASeg = MT / 8, kSeg = kBSeg + kASeg;   // 1 KB DMA segments per stage
  constexpr int kStage = kSeg * 1024;
  constexpr int kTM = MT >= 32 ? MT / 32 : 1, kTN = NT >= 32 ? NT / 32 : 1;   // MFMA tiles
  constexpr int kParts = dec_scale_parts(MT, NT);
  static_assert(NW * S * kStage <= kDecDataBytes, "stage rings exceed their LDS");
  static_assert(NW * kTM * kTN * 16 * 64 * 4 <= kDecDataBytes, "partials exceed the ring LDS");
  static_assert(kSeg * (S - 2) < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * NT, m0 = blockIdx.y * MT;
  const int kq = K / NW;                        // this wave's K range: [wave kq, (wave + 1) kq)
  const int J = kq / kDecStepK;                 // stages of the range
  const int kblocks = K / 32;
  uint8_t *wl = smem + wave * S * kStage;

  // DMA sources: segment i < kBSeg fills weight rows 8 i .. 8 i + 7 of a
  // stage, the others activation rows 8 (i - kBSeg) ..; lane l takes row
  // 8 i + l / 8 and fetches the global chunk (l % 8) ^ g(row), which lands
  // in slot l % 8.
  const uint8_t *src[kSeg];
#pragma unroll
  for (int i = 0; i < kSeg; ++i) {
    const int q = 8 * (i < kBSeg ? i : i - kBSeg) + (lane >> 3);
    const int c = (lane & 7) ^ dec_swz(q);
    const size_t row = i < kBSeg ? (size_t)min(n0 + q, N - 1) : (size_t)min(m0 + q, M - 1);
    src[i] = (i < kBSeg ? B : A) + row * (size_t)K + (size_t)wave * kq + c * 16;
  }
  auto issue = [&](int j) {
    uint8_t *dst = wl + (j % S) * kStage;
#pragma unroll
    for (int i = 0; i < kSeg; ++i) dma16(src[i] + j * kDecStepK, dst + i * 1024);
  };
  // Scale codes of the wave's range: 16-byte piece t of scale row q (q < NT:
  // weight row n0 + q, NT <= q < NT + MT: activation row m0 + q - NT; lanes
  // past the last row repeat a weight row) at sc + (t kParts + q / 64) KB +
  // (q % 64) * 16.
  const int pieces = kq / 512;
  uint8_t *sc = smem + kDecDataBytes + wave * pieces * kParts * 1024;
  if (MX) {
#pragma unroll
    for (int u = 0; u < kParts; ++u) {
      const int q = 64 * u + lane < NT + MT ? 64 * u + lane : 0;
      const uint8_t *ssrc = q < NT ? SB + (size_t)min(n0 + q, N - 1) * kblocks
                                   : SA + (size_t)min(m0 + q - NT, M - 1) * kblocks;
      ssrc += wave * (kq / 32);
      for (int t = 0; t < pieces; ++t) dma16(ssrc + 16 * t, sc + (t * kParts + u) * 1024);
    }
  }
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < J) issue(j);

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16{0};
  int brow[kTN], arow[kTM];
#pragma unroll
  for (int j = 0; j < kTN; ++j) brow[j] = NT >= 32 ? 32 * j + r : r % NT;
#pragma unroll
  for (int i = 0; i < kTM; ++i) arow[i] = MT >= 32 ? 32 * i + r : r % MT;
  auto frag = [&](const uint8_t *base, int row, int t) {
    const int g = dec_swz(row);
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + row * kDecStepK + (((4 * t + h) ^ g) << 4));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + row * kDecStepK + (((4 * t + 2 + h) ^ g) << 4));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto code = [&](int q, int blk) {
    return (int)sc[((blk >> 4) * kParts + (q >> 6)) * 1024 + (q & 63) * 16 + (blk & 15)];
  };
  for (int j = 0; j < J; ++j) {
    // stage j of this wave: the later stages already issued may stay in flight
    dec_wait<kSeg, S - 2>(min(J - 1, j + S - 2) - j);
    if (j + S - 1 < J) issue(j + S - 1);
    const uint8_t *st = wl + (j % S) * kStage;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int blk = 4 * j + 2 * t + h;        // 32-element block within the wave's range
      i32x8 bf[kTN], af[kTM];
      int sb[kTN], sa[kTM];
#pragma unroll
      for (int jj = 0; jj < kTN; ++jj) {
        bf[jj] = frag(st, brow[jj], t);
        sb[jj] = MX ? code(brow[jj], blk) : unit_scale;
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        af[i] = frag(st + kBSeg * 1024, arow[i], t);
        sa[i] = MX ? code(NT + arow[i], blk) : unit_scale;
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int jj = 0; jj < kTN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[jj], acc[i][jj], 0, 0, 0, sa[i],
                                                                       0, sb[jj]);
    }
  }

  // partials: red[((wave * kTM + i) * kTN + j) * 1024 + v * 64 + lane] over
  // the (now idle) stage rings
  __syncthreads();
  float *red = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int jj = 0; jj < kTN; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * kTM + i) * kTN + jj) * 1024 + v * 64 + lane] = acc[i][jj][v];
  __syncthreads();
  const float s = MX ? 1.0f : (*a_scale) * (*b_scale);
  constexpr int kOut = kTM * kTN * 1024;
  for (int e = tid; e < kOut; e += 64 * NW) {
    const int tile = e >> 10, v = (e >> 6) & 15, l = e & 63;
    const int tr = 32 * (tile / kTN) + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    const int tc = 32 * (tile % kTN) + (l & 31);
    const int row = m0 + tr, col = n0 + tc;
    if (tr < MT && tc < NT && row < M && col < N) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w * kOut + e];
      C[(size_t)row * (size_t)N + col] = (uint16_t)(Bf16::pack(sum * s, 0.0f) & 0xffffu);
    }
  }
}

#define GNQ_GEMM_DEC_INST(MX, NW, MT, NT, S)                                                      \
  template __global__ void gemm_fp8_decode<MX, NW, MT, NT, S>(                                    \
      const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *, const float *,         \
      const float *, int, int, int, uint16_t *, int);
GNQ_GEMM_DEC_INST(true, 4, 32, 16, 5)
GNQ_GEMM_DEC_INST(false, 4, 32, 16, 5)
GNQ_GEMM_DEC_INST(true, 4, 32, 32, 4)
GNQ_GEMM_DEC_INST(false, 4, 32, 32, 4)
GNQ_GEMM_DEC_INST(true, 2, 64, 64, 4)
GNQ_GEMM_DEC_INST(false, 2, 64, 64, 4)
#undef GNQ_GEMM_DEC_INST

template <bool MX, int NW, int MT, int NT, int S>
hipError_t launch_decode_tile(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                              const float *a_scale, const float *b_scale, int M, int N, int K, uint16_t *C,
                              hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = allow_dynamic_lds((const void *)gemm_fp8_decode<MX, NW, MT, NT, S>, kDecLdsMax, lds_set);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((N + NT - 1) / NT), (unsigned)((M + MT - 1) / MT));
  return launch(gemm_fp8_decode<MX, NW, MT, NT, S>, grid, dim3(64 * NW), dec_lds_bytes(K, MT, NT), st, A,
                SA, B, SB, a_scale, b_scale, M, N, K, C, 127);
}

// Tile choice (measured on 4096- and 8192-wide weights, K 4096 and 8192):
// 64 x 64 with 2 waves when that still gives >= 256 workgroups (M = 256:
// 20-30% faster than 32 x 32, which re-reads both operands twice as often;
// it needs K <= 8192 for its scale slab); else 32 x 32 unless that leaves
// fewer than 192 workgroups, then 32 x 16.  8-row tiles with deeper rings
// measured no faster for one row: the weight stream already runs at the HBM
// rate past a fixed ~3 us of launch, first round trip and reduction.
template <bool MX>
hipError_t launch_decode(const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                         const float *a_scale, const float *b_scale, int M, int N, int K, uint16_t *C,
                         hipStream_t st) {
  const long wide = (long)((N + 63) / 64) * ((M + 63) / 64);
  if (K <= 8192 && wide >= 256)
    return launch_decode_tile<MX, 2, 64, 64, 4>(A, SA, B, SB, a_scale, b_scale, M, N, K, C, st);
  const long mid = (long)((N + 31) / 32) * ((M + 31) / 32);
  if (mid < 192) return launch_decode_tile<MX, 4, 32, 16, 5>(A, SA, B, SB, a_scale, b_scale, M, N, K, C, st);
  return launch_decode_tile<MX, 4, 32, 32, 4>(A, SA, B, SB, a_scale, b_scale, M, N, K, C, st);
}

// NVFP4 consumer: C[M, N] = dq(A) dq(B)^T in bf16 for the op's NVFP4 output
// as it stands (E2M1 codes, element 2 j in the low nibble of byte j; E4M3
// block scales per 16 elements in the 128x4-tiled buffer; dq = code x scale
// / gs).  The block-scaled MFMA takes only power-of-two (E8M0) scales, and a
// code times an E4M3 scale has up to 5 significant bits (not exact in any
// 8-bit format), so the operands are dequantized exactly to fp16 (11
// significant bits; every such product lies in fp16's normal range) in
// registers and fed to the fp16 MFMA (v_mfma_f32_32x32x16_f16; its operand
// and accumulator layout, measured with a one-wave probe, match the
// block-scaled one's for rows and outputs); 1 / (gs_a gs_b) is applied to
// the fp32 sum.  The hardware's scaled E2M1 -> fp16 conversion applies only
// the exponent of its scale (probe), so a block scale is split into a power
// of two for the conversion and a 3-bit significand applied by one packed
// fp16 multiply per two elements (fp4x8_f16 below).
//
// Structure of the decode kernel: a workgroup owns an MT x NT tile, its NW
// waves split K into contiguous ranges, each streaming its range through a
// private ring of S LDS stages (64 K-elements: 32 code bytes per row and the
// 512-byte scale chunk of the 128-row scale tile) by 16-byte DMA, with no
// barrier; the partial tiles are summed through LDS in a fixed order.
// A lane's 16 K-elements per half stage are one whole block (lanes 0..31
// block 2 j, lanes 32..63 block 2 j + 1), read as 8 bytes; every element is
// scaled by its own block's scale before the MFMA, so the MFMA's pairing of
// K positions need not follow the blocks.  Code rows are 32 bytes; their
// 16-byte halves are swapped on every other group of 8 rows (g(q) =
// (q / 8) % 2) to halve the LDS bank conflicts of those reads.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
constexpr int kFp4StepK = 64;                       // K elements per stage
constexpr int kFp4StepBytes = kFp4StepK / 2;        // code bytes per row per stage
constexpr int kFp4ScaleChunk = 512;                 // 128 rows x 4 blocks of scales

__device__ __forceinline__ int fp4_swz(int row) { return (row >> 3) & 1; }

// 8 E2M1 codes (element 2 j in the low nibble of byte j) times their block
// scale, as 8 fp16 (exact: a code times an E4M3 scale has at most 5
// significant bits and lies within fp16's normal range).  The hardware's
// packed FP4 -> fp16 conversion (v_cvt_scalef32_pk_f16_fp4; operand byte j
// gives elements 2 j, 2 j + 1, low nibble first) applies only the exponent
// of its fp32 scale operand (probed: 1.125, 1.5 and 1.875 act as 1, 3 as 2,
// 2^-9 and 448 as 2^-9 and 256), so it is passed `sig` for the power of two
// and the packed fp16 multiply by `mant` supplies the significand
// (fp4_block_scale).  Intermediates stay normal: code x 2^E lies in
// [2^-9, 3072] for E4M3 scales.
__device__ __forceinline__ f16x8 fp4x8_f16(uint32_t w, float sig, f16x2 mant) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sig, 0) * mant;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sig, 1) * mant;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sig, 2) * mant;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sig, 3) * mant;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Splits a block scale v (the fp32 value of its E4M3 byte) as v = M 2^E,
// M = frexp mantissa in [0.5, 1) with v's sign: `mant` = M as a packed fp16
// pair (exact, 3 significant bits) and `sig` = 2 |v|, whose exponent field is
// E.  A zero scale gives M = 0 and a NaN scale M = NaN, so the products come
// out as the plain multiply gives them.
__device__ __forceinline__ void fp4_block_scale(float v, float &sig, f16x2 &mant) {
  sig = __builtin_fabsf(v) + __builtin_fabsf(v);
  const _Float16 mh = (_Float16)__builtin_amdgcn_frexp_mantf(v);
  mant = f16x2{mh, mh};
}

// Workgroup b runs on XCD b % 8: give each XCD a contiguous range of the
// n workgroups' tiles, so the workgroups that share a 128-row scale tile
// share one L2 (a bijection on 0 .. n - 1).
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
  const int q = n / kXcds, r = n % kXcds, x = b % kXcds;
  return x * q + min(x, r) + b / kXcds;
}

template <int NW, int MT, int NT, int S>
__global__ void __launch_bounds__(64 * NW)
gemm_nvfp4_k(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ a_gs,
             const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ b_gs,
             int M, int N, int K, uint16_t *__restrict__ C, int tiles_n) {
  constexpr int kBSeg = NT / 32, kASeg = MT / 32, kCSeg = kBSeg + kASeg;   // 1 KB code segments
  constexpr int kCodeB = NT * kFp4StepBytes, kCodeA = MT * kFp4StepBytes;
  constexpr int kStage = kCodeB + kCodeA + 2 * kFp4ScaleChunk;
  constexpr int kTM = MT / 32, kTN = NT / 32;
  static_assert(MT % 32 == 0 && NT % 32 == 0 && 128 % MT == 0 && 128 % NT == 0, "tiles inside one scale tile");
  static_assert(NW * S * kStage <= kDecDataBytes, "stage rings exceed their LDS");
  static_assert(NW * kTM * kTN * 4096 <= kDecDataBytes, "partials exceed the LDS");
  static_assert((kCSeg + 1) * (S - 2) < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int bt = xcd_contiguous(blockIdx.x, gridDim.x);   // consecutive weight tiles on one XCD
  const int tm = bt / tiles_n, tn = bt % tiles_n;
  const int m0 = tm * MT, n0 = tn * NT;
  const int ksteps = K / kFp4StepK;             // stages over all of K
  // this wave's stages: j0 .. j0 + J - 1 (an even split; J may be 0)
  const int j0 = (wave * ksteps) / NW;
  const int J = ((wave + 1) * ksteps) / NW - j0;
  const size_t rowb = (size_t)K / 2;
  uint8_t *wl = smem + wave * S * kStage;

  // Code segment i (< kBSeg: weight rows 32 i .., else activation rows):
  // lane l takes row 32 i + l / 2 and fetches the global half (l % 2) ^ g(row),
  // landing at half l % 2 of the row's 32 LDS bytes.
  const uint8_t *src[kCSeg];
#pragma unroll
  for (int i = 0; i < kCSeg; ++i) {
    const int q = 32 * (i < kBSeg ? i : i - kBSeg) + (lane >> 1);
    const size_t row = i < kBSeg ? (size_t)min(n0 + q, N - 1) : (size_t)min(m0 + q, M - 1);
    src[i] = (i < kBSeg ? B : A) + row * rowb + (size_t)j0 * kFp4StepBytes + 16 * ((lane & 1) ^ fp4_swz(q));
  }
  // Scale chunk of stage j: lanes 0..31 the weight's 512 bytes, 32..63 the
  // activation's, each 16 bytes.
  const uint8_t *ssrc = lane < 32 ? SB + ((size_t)(n0 / 128) * ksteps + (size_t)j0) * kFp4ScaleChunk + 16 * lane
                                  : SA + ((size_t)(m0 / 128) * ksteps + (size_t)j0) * kFp4ScaleChunk + 16 * (lane - 32);
  auto issue = [&](int j) {
    uint8_t *dst = wl + (j % S) * kStage;
#pragma unroll
    for (int i = 0; i < kCSeg; ++i)
      dma16(src[i] + (size_t)j * kFp4StepBytes, dst + (i < kBSeg ? i * 1024 : kCodeB + (i - kBSeg) * 1024));
    dma16(ssrc + (size_t)j * kFp4ScaleChunk, dst + kCodeB + kCodeA);
  };
#pragma unroll
  for (int j = 0; j < S - 1; ++j)
    if (j < J) issue(j);

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int jj = 0; jj < kTN; ++jj) acc[i][jj] = f32x16{0};
  // rows of this lane's fragments inside the tile and inside the 128-row scale tile
  const int bq0 = r, aq0 = r;
  const int bs0 = n0 % 128, as0 = m0 % 128;
  for (int j = 0; j < J; ++j) {
    dec_wait<kCSeg + 1, S - 2>(min(J - 1, j + S - 2) - j);
    if (j + S - 1 < J) issue(j + S - 1);
    const uint8_t *st = wl + (j % S) * kStage;
    const uint8_t *sch = st + kCodeB + kCodeA;
#pragma unroll
    for (int p = 0; p < 2; ++p) {                 // half stage: blocks 2 p (lanes 0..31), 2 p + 1 (32..63)
      const int blk = 2 * p + h;
      f16x8 bf[kTN][2], af[kTM][2];
#pragma unroll
      for (int jj = 0; jj < kTN; ++jj) {
        const int q = 32 * jj + bq0, qs = bs0 + q;
        const uint2 w = *reinterpret_cast<const uint2 *>(st + q * kFp4StepBytes + 16 * (p ^ fp4_swz(q)) + 8 * h);
        float sig;
        f16x2 mant;
        fp4_block_scale(__builtin_amdgcn_cvt_f32_fp8((int)sch[(qs & 31) * 16 + (qs >> 5) * 4 + blk], 0), sig, mant);
        bf[jj][0] = fp4x8_f16(w.x, sig, mant);
        bf[jj][1] = fp4x8_f16(w.y, sig, mant);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i) {
        const int q = 32 * i + aq0, qs = as0 + q;
        const uint2 w = *reinterpret_cast<const uint2 *>(st + kCodeB + q * kFp4StepBytes + 16 * (p ^ fp4_swz(q)) + 8 * h);
        float sig;
        f16x2 mant;
        fp4_block_scale(__builtin_amdgcn_cvt_f32_fp8((int)sch[kFp4ScaleChunk + (qs & 31) * 16 + (qs >> 5) * 4 + blk], 0),
                        sig, mant);
        af[i][0] = fp4x8_f16(w.x, sig, mant);
        af[i][1] = fp4x8_f16(w.y, sig, mant);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int jj = 0; jj < kTN; ++jj)
            acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i][e], bf[jj][e], acc[i][jj], 0, 0, 0);
    }
  }

  __syncthreads();
  float *red = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int jj = 0; jj < kTN; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[((wave * kTM + i) * kTN + jj) * 1024 + v * 64 + lane] = acc[i][jj][v];
  __syncthreads();
  const float s = 1.0f / ((*a_gs) * (*b_gs));
  constexpr int kOut = kTM * kTN * 1024;
  for (int e = tid; e < kOut; e += 64 * NW) {
    const int tile = e >> 10, v = (e >> 6) & 15, l = e & 63;
    const int row = m0 + 32 * (tile / kTN) + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    const int col = n0 + 32 * (tile % kTN) + (l & 31);
    if (row < M && col < N) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w * kOut + e];
      C[(size_t)row * (size_t)N + col] = (uint16_t)(Bf16::pack(sum * s, 0.0f) & 0xffffu);
    }
  }
}

#define GNQ_GEMM_FP4_INST(NW, MT, NT, S)                                                          \
  template __global__ void gemm_nvfp4_k<NW, MT, NT, S>(const uint8_t *, const uint8_t *, const float *, \
                                                        const uint8_t *, const uint8_t *, const float *, int, \
                                                        int, int, uint16_t *, int);
GNQ_GEMM_FP4_INST(4, 32, 32, 8)
GNQ_GEMM_FP4_INST(8, 32, 32, 4)
GNQ_GEMM_FP4_INST(8, 64, 32, 4)
GNQ_GEMM_FP4_INST(8, 64, 64, 3)
GNQ_GEMM_FP4_INST(4, 128, 64, 4)
#undef GNQ_GEMM_FP4_INST

// Many rows: 256 x 256 workgroup tiles (4 waves of 128 x 128, 16 MFMA tiles
// each), operands staged in shared LDS stages of 64 K-elements by 16-byte
// DMA (codes of 256 + 256 rows and the four 512-byte scale tiles of their
// two 128-row groups), one barrier per stage.  Each converted fragment feeds
// 4 MFMAs instead of 2 in a 64 x 64 tile, halving the dequantization per
// MFMA.  Scale tiles past the last 128-row group (a partial 256-row tile)
// are not read: the last group's tile stands in, for rows whose outputs are
// dropped.
constexpr int kFp4BigRows = 256;
constexpr int kFp4BigStages = 6;
constexpr int kFp4BigCode = kFp4BigRows * kFp4StepBytes;                 // 8 KB per operand
constexpr int kFp4BigStage = 2 * kFp4BigCode + 4 * kFp4ScaleChunk;       // + A lo/hi, B lo/hi scale tiles
constexpr int kFp4BigLds = kFp4BigStages * kFp4BigStage;                 // 108 KB

__global__ void __launch_bounds__(256)
gemm_nvfp4_big(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ a_gs,
               const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ b_gs,
               int M, int N, int K, uint16_t *__restrict__ C, int tiles_m, int tiles) {
  constexpr int kPer = 5;                               // DMA instructions per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, h = lane >> 5;
  int tm, tn;
  gemm_tile_of_block(blockIdx.x, tiles_m, tiles / tiles_m, tm, tn);
  const int m0 = tm * kFp4BigRows, n0 = tn * kFp4BigRows;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  const int ksteps = K / kFp4StepK;
  const size_t rowb = (size_t)K / 2;

  // Code segments: wave w fetches 1 KB segments 4 w .. 4 w + 3 of the
  // stage's 16 (0..7: A rows 32 i .., 8..15: B rows); lane l takes row
  // 32 i + l / 2, global half (l % 2) ^ g(row) into half l % 2.
  const uint8_t *src[4];
  int dsto[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int seg = 4 * wave + t;
    const bool isb = seg >= 8;
    const int q = 32 * (seg & 7) + (lane >> 1);
    const size_t row = isb ? (size_t)min(n0 + q, N - 1) : (size_t)min(m0 + q, M - 1);
    src[t] = (isb ? B : A) + row * rowb + 16 * ((lane & 1) ^ fp4_swz(q));
    dsto[t] = (isb ? kFp4BigCode : 0) + (seg & 7) * 1024;
  }
  // Scale tiles: wave w fetches tile w (0, 1: A's two 128-row groups; 2, 3:
  // B's) with lanes 0..31, 16 bytes each.
  const bool sb_ = wave >= 2;
  const int groups = sb_ ? (N + 127) / 128 : (M + 127) / 128;
  const int grp = min((sb_ ? n0 : m0) / 128 + (wave & 1), groups - 1);
  const uint8_t *ssrc = (sb_ ? SB : SA) + (size_t)grp * ksteps * kFp4ScaleChunk + 16 * (lane & 31);
  const int sdst = 2 * kFp4BigCode + wave * kFp4ScaleChunk;
  auto issue = [&](int ks, int from) {
    uint8_t *st = smem + (ks % kFp4BigStages) * kFp4BigStage;
#pragma unroll
    for (int t = 0; t < 4; ++t) dma16(src[t] + (size_t)from * kFp4StepBytes, st + dsto[t]);
    if (lane < 32) dma16(ssrc + (size_t)from * kFp4ScaleChunk, st + sdst);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{0};

  // K pairing: lanes of half h (lanes 32 h .. 32 h + 31) take global chunk h
  // of a row's 64-element step, blocks 2 h and 2 h + 1; half stage p feeds
  // block 2 h + p to the 32 MFMAs (two of K 16 per tile) of that half.  A
  // step's fragments -- 8 rows (4 of A, 4 of B) of 16 code bytes and the two
  // scale bytes of those blocks -- are read into one of two buffers during
  // the half stage before their first conversion, so the LDS latency runs
  // beside the MFMAs.  Within a 32-row slice the lane's offsets are the same for every
  // fragment (the chunk swizzle depends on the row's bits 3 only).
  const int lane_code = r * kFp4StepBytes + 16 * (h ^ fp4_swz(r));
  const int lane_scale = r * 16 + 2 * h;
  uint4 raw[2][8];
  uint32_t scw[2][8];
  f16x8 fr[2][8][2];
  // Read item t of step ks into buffer `buf`: fragment t / 2, its codes
  // (t even) or its scale bytes (t odd).
  auto read_item = [&](int buf, int ks, int t) {
    const uint8_t *st = smem + (ks % kFp4BigStages) * kFp4BigStage;
    const int f = t >> 1;
    const bool isb = f >= 4;
    const int q0 = (isb ? wn : wm) + 32 * (f & 3);
    if ((t & 1) == 0)
      raw[buf][f] = *reinterpret_cast<const uint4 *>(st + (isb ? kFp4BigCode : 0) + q0 * kFp4StepBytes + lane_code);
    else
      scw[buf][f] = *reinterpret_cast<const uint16_t *>(st + 2 * kFp4BigCode +
                                                        ((isb ? 2 : 0) + (q0 >> 7)) * kFp4ScaleChunk + (f & 3) * 4 +
                                                        lane_scale);
  };
  // Conversion unit u of half stage p from buffer `buf`: fragment u / 2,
  // MFMA half u % 2 (8 elements), into register set `set`.
  float sig;
  f16x2 mant;
  auto convert = [&](int set, int buf, int p, int u) {
    const int f = u >> 1;
    if ((u & 1) == 0)
      fp4_block_scale(p ? __builtin_amdgcn_cvt_f32_fp8((int)scw[buf][f], 1) : __builtin_amdgcn_cvt_f32_fp8((int)scw[buf][f], 0),
                      sig, mant);
    const uint32_t w = p ? ((u & 1) ? raw[buf][f].w : raw[buf][f].z) : ((u & 1) ? raw[buf][f].y : raw[buf][f].x);
    fr[set][f][u & 1] = fp4x8_f16(w, sig, mant);
  };
  // MFMAs of register set `set`, with the 16 conversion units of the next
  // half stage (buffer `buf`, half `np`, into the other set) between them,
  // one after every second MFMA, so the VALU dequantization runs beside the
  // MFMA pipe; with `rd`, the 16 read items of step `rks` into buffer `rbuf`
  // go between the others, spread so that the four waves' LDS reads do not
  // arrive as one burst.
  auto half = [&](int set, int buf, int np, bool rd, int rbuf, int rks) {
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int e = q >> 4, i = (q >> 2) & 3, j = q & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[set][i][e], fr[set][4 + j][e], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (q & 1)
        convert(set ^ 1, buf, np, q >> 1);
      else if (rd)
        read_item(rbuf, rks, q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Step ks from buffer `cur`; step ks + 1 (landed, per the wait) is read
  // into buffer `nxt` during the first half.  A plain barrier (a fenced one would drain all DMA in
  // flight): every read of stage ks - 1 happened before it, so its slot can
  // be refilled; refetches past the end keep the DMA count uniform.
  auto step = [&](int ks, int cur, int nxt) {
    wait_vmcnt<kPer * (kFp4BigStages - 3)>();
    asm volatile("s_barrier" ::: "memory");
    issue(ks + kFp4BigStages - 1, min(ks + kFp4BigStages - 1, ksteps - 1));
    half(0, cur, 1, true, nxt, ks + 1);   // MFMAs of (ks, 0), conversion of (ks, 1), reads of ks + 1
    half(1, nxt, 0, false, 0, 0);         // MFMAs of (ks, 1), conversion of (ks + 1, 0)
  };

#pragma unroll
  for (int j = 0; j < kFp4BigStages - 1; ++j) issue(j, min(j, ksteps - 1));
  wait_vmcnt<kPer * (kFp4BigStages - 2)>();
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int t = 0; t < 16; ++t) read_item(0, 0, t);
#pragma unroll
  for (int u = 0; u < 16; ++u) convert(0, 0, 0, u);
  int ks = 0;
  for (; ks + 1 < ksteps; ks += 2) {
    step(ks, 0, 1);
    step(ks + 1, 1, 0);
  }
  if (ks < ksteps) step(ks, 0, 1);             // odd step count
  wait_vmcnt<0>();   // the refetches land before the workgroup's LDS is released

  const float s = 1.0f / ((*a_gs) * (*b_gs));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + 32 * j + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < M && col < N)
          C[(size_t)row * (size_t)N + col] = (uint16_t)(Bf16::pack(acc[i][j][v] * s, 0.0f) & 0xffffu);
      }
    }
}

hipError_t launch_nvfp4_big(const uint8_t *A, const uint8_t *SA, const float *a_gs, const uint8_t *B,
                            const uint8_t *SB, const float *b_gs, int M, int N, int K, uint16_t *C, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = allow_dynamic_lds((const void *)gemm_nvfp4_big, kFp4BigLds, lds_set);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + kFp4BigRows - 1) / kFp4BigRows, tiles_n = (N + kFp4BigRows - 1) / kFp4BigRows;
  const int tiles = tiles_m * tiles_n;
  return launch(gemm_nvfp4_big, dim3((unsigned)tiles), dim3(256), kFp4BigLds, st, A, SA, a_gs, B, SB, b_gs, M,
                N, K, C, tiles_m, tiles);
}

template <int NW, int MT, int NT, int S>
hipError_t launch_nvfp4(const uint8_t *A, const uint8_t *SA, const float *a_gs, const uint8_t *B,
                        const uint8_t *SB, const float *b_gs, int M, int N, int K, uint16_t *C, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  // the stage rings, or the partial tiles summed over them at the end
  constexpr int ring = NW * S * (NT * kFp4StepBytes + MT * kFp4StepBytes + 2 * kFp4ScaleChunk);
  constexpr int part = NW * (MT / 32) * (NT / 32) * 4096;
  constexpr int lds = ring > part ? ring : part;
  const hipError_t e = allow_dynamic_lds((const void *)gemm_nvfp4_k<NW, MT, NT, S>, lds, lds_set);
  if (e != hipSuccess) return e;
  const int tiles_n = (N + NT - 1) / NT;
  const long tiles = (long)((M + MT - 1) / MT) * tiles_n;
  return launch(gemm_nvfp4_k<NW, MT, NT, S>, dim3((unsigned)tiles), dim3(64 * NW), lds, st, A, SA, a_gs, B,
                SB, b_gs, M, N, K, C, tiles_n);
}

// Few activation rows (up to 8): a dot-product kernel, since 32-row MFMA
// tiles would dequantize a mostly padded activation tile for every weight
// tile.  The workgroup first dequantizes the activation once into LDS as
// fp16 (row m, 32-element chunk ci at (m * K / 32 + ci) * 80 bytes: the
// 16-byte pad puts the chunks that 16 consecutive lanes read on distinct
// banks).  Its 8 waves own 16 weight rows, two per wave (lanes 0..31 and
// 32..63); lane c of a row takes the row's 16-byte code chunks c, c + 32, ...
// (32 elements: blocks 2 ci and 2 ci + 1, their two scale bytes adjacent in
// the tiled buffer), loaded four ahead of their use; the row blocks are laid
// out contiguously per XCD (xcd_contiguous).  A block's 16 codes are
// converted at the power of two of its scale (fp4_block_scale), dotted with
// each activation row by v_dot2_f32_f16 into a block sum (exact products,
// fp32 sums), and the block's significand multiplies that sum into the row's
// accumulator.  The 32 lanes' sums of a row meet in a butterfly.
constexpr int kGemvRows = 16;             // weight rows per workgroup
constexpr int kGemvChunk = 80;            // LDS bytes per 32-element activation chunk
constexpr int kGemvMaxLds = 128 * 1024;
constexpr int kGemvGroup = 4;             // weight chunks per lane in flight

__device__ __forceinline__ size_t nvfp4_scale_offset(int row, int blk, int kp4) {
  // byte of (row, 16-element block) in the 128x4-tiled buffer, kp4 = K / 64
  return ((size_t)(row >> 7) * kp4 + (blk >> 2)) * 512 + (row & 31) * 16 + ((row & 127) >> 5) * 4 + (blk & 3);
}

template <int MR>
__global__ void __launch_bounds__(512)
gemm_nvfp4_gemv(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ a_gs,
                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ b_gs,
                int M, int N, int K, uint16_t *__restrict__ C) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = K / 32, kp4 = K / 64;
  const int c = lane & 31;
  const int row = xcd_contiguous(blockIdx.x, gridDim.x) * kGemvRows + 2 * wave + (lane >> 5);
  const int rowc = min(row, N - 1);
  const uint8_t *brow = B + (size_t)rowc * (size_t)(K / 2);

  uint4 code[2][kGemvGroup];
  uint32_t scw[2][kGemvGroup];
  // chunks c + 32 (g + j) of group g; past the row's end the last chunk is
  // refetched (in bounds) and its contribution skipped
  auto load = [&](int buf, int g) {
#pragma unroll
    for (int j = 0; j < kGemvGroup; ++j) {
      const int ci = min(c + 32 * (g + j), nch - 1);
      code[buf][j] = *reinterpret_cast<const uint4 *>(brow + (size_t)ci * 16);
      scw[buf][j] = *reinterpret_cast<const uint16_t *>(SB + nvfp4_scale_offset(rowc, 2 * ci, kp4));
    }
  };
  load(0, 0);

  // the activation, dequantized (code x block scale; 1 / gs comes last)
  const int units = M * (K / 8);
  for (int u = tid; u < units; u += 512) {
    const int m = u / (K / 8), k = (u - m * (K / 8)) * 8;
    const uint32_t w = *reinterpret_cast<const uint32_t *>(A + (size_t)m * (size_t)(K / 2) + k / 2);
    float sig;
    f16x2 mant;
    fp4_block_scale(__builtin_amdgcn_cvt_f32_fp8((int)SA[nvfp4_scale_offset(m, k / 16, kp4)], 0), sig, mant);
    *reinterpret_cast<f16x8 *>(smem + ((size_t)m * nch + k / 32) * kGemvChunk + (k % 32) * 2) =
        fp4x8_f16(w, sig, mant);
  }
  __syncthreads();

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
  const int groups = (nch + 31) / 32;          // chunk groups of 32 per row, kGemvGroup at a time
  for (int g = 0; g < groups; g += 2 * kGemvGroup) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int gg = g + half * kGemvGroup;
      if (gg >= groups) break;
      if (gg + kGemvGroup < groups) load(half ^ 1, gg + kGemvGroup);
#pragma unroll
      for (int j = 0; j < kGemvGroup; ++j) {
        const int ci = c + 32 * (gg + j);
        if (ci >= nch) continue;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const float v = blk ? __builtin_amdgcn_cvt_f32_fp8((int)scw[half][j], 1)
                              : __builtin_amdgcn_cvt_f32_fp8((int)scw[half][j], 0);
          const float sig = __builtin_fabsf(v) + __builtin_fabsf(v);
          const float mant = __builtin_amdgcn_frexp_mantf(v);
          const uint32_t w0 = blk ? code[half][j].z : code[half][j].x;
          const uint32_t w1 = blk ? code[half][j].w : code[half][j].y;
          f16x2 bp[8];
          bp[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, sig, 0);
          bp[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, sig, 1);
          bp[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, sig, 2);
          bp[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, sig, 3);
          bp[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, sig, 0);
          bp[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, sig, 1);
          bp[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, sig, 2);
          bp[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, sig, 3);
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            if (m >= M) break;
            const uint8_t *ap = smem + ((size_t)m * nch + ci) * kGemvChunk + blk * 32;
            const uint4 a0 = *reinterpret_cast<const uint4 *>(ap);
            const uint4 a1 = *reinterpret_cast<const uint4 *>(ap + 16);
            float t = 0.0f;
            t = __builtin_amdgcn_fdot2(bp[0], __builtin_bit_cast(f16x2, a0.x), t, false);
            t = __builtin_amdgcn_fdot2(bp[1], __builtin_bit_cast(f16x2, a0.y), t, false);
            t = __builtin_amdgcn_fdot2(bp[2], __builtin_bit_cast(f16x2, a0.z), t, false);
            t = __builtin_amdgcn_fdot2(bp[3], __builtin_bit_cast(f16x2, a0.w), t, false);
            t = __builtin_amdgcn_fdot2(bp[4], __builtin_bit_cast(f16x2, a1.x), t, false);
            t = __builtin_amdgcn_fdot2(bp[5], __builtin_bit_cast(f16x2, a1.y), t, false);
            t = __builtin_amdgcn_fdot2(bp[6], __builtin_bit_cast(f16x2, a1.z), t, false);
            t = __builtin_amdgcn_fdot2(bp[7], __builtin_bit_cast(f16x2, a1.w), t, false);
            acc[m] = __builtin_fmaf(t, mant, acc[m]);
          }
        }
      }
    }
  }

  const float s = 1.0f / ((*a_gs) * (*b_gs));
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m >= M) break;
    float v = acc[m];
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (c == 0 && row < N) C[(size_t)m * (size_t)N + row] = (uint16_t)(Bf16::pack(v * s, 0.0f) & 0xffffu);
  }
}

template <int MR>
hipError_t launch_nvfp4_gemv(const uint8_t *A, const uint8_t *SA, const float *a_gs, const uint8_t *B,
                             const uint8_t *SB, const float *b_gs, int M, int N, int K, uint16_t *C, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = allow_dynamic_lds((const void *)gemm_nvfp4_gemv<MR>, kGemvMaxLds, lds_set);
  if (e != hipSuccess) return e;
  const int lds = M * (K / 32) * kGemvChunk;
  return launch(gemm_nvfp4_gemv<MR>, dim3((unsigned)((N + kGemvRows - 1) / kGemvRows)), dim3(512), lds, st,
                A, SA, a_gs, B, SB, b_gs, M, N, K, C);
}

// Caller guarantees K % 64 == 0, 0 < M, N, and that the 32 x 32 tile count
// fits a grid.  Tile choice (measured at N = 4096 and 8192, K = 4096): a
// workgroup round costs about the same whatever its tile, so the largest
// tile that still gives enough workgroups wins.  For a few rows against a
// narrow weight (M <= 8, M N <= 12288) the dot-product kernel; beyond 256 rows the 256 x 256 kernel once it has 128
// workgroups (at N = 4096 it took 108 us at M = 300 to 1024 with 32-64
// workgroups, against 31-67 us on 128 x 64 tiles); else the first of
// 128 x 64, 64 x 64, 64 x 32 tiles giving 192 workgroups (M = 200: 64 x 64
// 19.4 us, 32 x 32 35.3 us); else 32 x 32 tiles.
hipError_t gemm_nvfp4(const void *a, const void *sa, const float *a_gs, const void *b, const void *sb,
                      const float *b_gs, int64_t M, int64_t N, int64_t K, void *c, hipStream_t st) {
  const uint8_t *A = (const uint8_t *)a, *B = (const uint8_t *)b;
  const uint8_t *SA = (const uint8_t *)sa, *SB = (const uint8_t *)sb;
  uint16_t *C = (uint16_t *)c;
  const int m = (int)M, n = (int)N, k = (int)K;
  // dot products while their work (M N dot products per K) stays below the
  // MFMA kernel's fixed cost: measured at N = K = 4096 they win up to
  // M = 3 (6.6 against 7.2 us) and lose from M = 4 (7.7 against 7.2, 12.3
  // against 7.3 at M = 8); at N = 8192 they tie at M = 2; the activation
  // must fit the LDS
  if (M <= 8 && M * N <= 12288 && M * (K / 32) * (int64_t)kGemvChunk <= kGemvMaxLds) {
    if (M == 1) return launch_nvfp4_gemv<1>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
    if (M == 2) return launch_nvfp4_gemv<2>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
    if (M <= 4) return launch_nvfp4_gemv<4>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
    return launch_nvfp4_gemv<8>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  }
  auto tiles = [&](int64_t mt, int64_t nt) { return ((M + mt - 1) / mt) * ((N + nt - 1) / nt); };
  if (M > 256 && tiles(kFp4BigRows, kFp4BigRows) >= 128)
    return launch_nvfp4_big(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  if (M >= 128 && tiles(128, 64) >= 192)
    return launch_nvfp4<4, 128, 64, 4>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  if (M >= 64 && tiles(64, 64) >= 192)
    return launch_nvfp4<8, 64, 64, 3>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  if (M >= 64 && tiles(64, 32) >= 192)
    return launch_nvfp4<8, 64, 32, 4>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  // 32 x 32 tiles; 8 waves splitting K when it divides into 8 equal ranges,
  // else 4 (ranges may differ by a stage)
  if (K % 512 == 0) return launch_nvfp4<8, 32, 32, 4>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
  return launch_nvfp4<4, 32, 32, 8>(A, SA, a_gs, B, SB, b_gs, m, n, k, C, st);
}

hipError_t gemm_fp8(bool mx, const void *a, const void *sa, const void *b, const void *sb,
                    const float *a_scale, const float *b_scale, int64_t M, int64_t N, int64_t K,
                    void *c, hipStream_t st) {
  const uint8_t *A = (const uint8_t *)a, *B = (const uint8_t *)b;
  const uint8_t *SA = (const uint8_t *)sa, *SB = (const uint8_t *)sb;
  // Tile choice (measured at N = 4096 and 8192, K = 4096): a workgroup's
  // 256 x 256 tile keeps one CU busy ~40 us, so with fewer than 128 such
  // workgroups the 128 x 128 tiles (four times as many, two workgroups per
  // CU) win: M = 300, 512, 1024 at N = 4096 took 41, 43, 46 us on 256 x 256
  // and 19, 21, 26 us on 128 x 128 (MXFP8); at 128 workgroups they tie.  Up
  // to 256 rows the decode kernel's small tiles stream the weight faster,
  // unless 128 x 128 tiles already number 128 (M = 192, N = 8192: 28.8 us
  // against 21.2 us).  The DMA pipeline needs K % 512 == 0 (a 16-byte scale
  // window never crosses a row of K / 32 codes) and 16-byte aligned scales.
  const bool dma = K % 512 == 0 && (!mx || ((uintptr_t)sa % 16 == 0 && (uintptr_t)sb % 16 == 0));
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256), t128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (dma && t256 >= 128)
    return mx ? launch_dma<true, 8, 2, 4, 256>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K,
                                               (uint16_t *)c, st)
              : launch_dma<false, 8, 2, 4, 256>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K,
                                                (uint16_t *)c, st);
  if (dma && (M > 256 || t128 >= 128))
    return mx ? launch_dma<true, 4, 2, 2, 128>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K,
                                               (uint16_t *)c, st)
              : launch_dma<false, 4, 2, 2, 128>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K,
                                                (uint16_t *)c, st);
  // Few activation rows: the decode kernel (or, for K it does not take, the
  // skinny one) streams the weight with small tiles.
  if (M <= 256 && K % 2048 == 0 && K <= kDecMaxK && (!mx || ((uintptr_t)sa % 16 == 0 && (uintptr_t)sb % 16 == 0)))
    return mx ? launch_decode<true>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K, (uint16_t *)c, st)
              : launch_decode<false>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K, (uint16_t *)c, st);
  if (M <= 256 && K % kGemmK == 0)
    return mx ? launch_skinny<true>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K, (uint16_t *)c, st)
              : launch_skinny<false>(A, SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K, (uint16_t *)c, st);
  const int tiles_m = (int)((M + kGemmTile - 1) / kGemmTile);
  const int tiles = tiles_m * (int)((N + kGemmTile - 1) / kGemmTile);
  return launch(mx ? gemm_fp8_tn<true> : gemm_fp8_tn<false>, dim3(tiles), dim3(kGemmThreads), 0, st, A,
                SA, B, SB, a_scale, b_scale, (int)M, (int)N, (int)K, (uint16_t *)c, tiles_m, tiles, 127);
}

}  // namespace gnq
