// Drives the C ABI's host-side argument checks (gnq_validate.hpp), built on
// their own with the address and undefined-behaviour sanitizers (see
// tests/test_host_sanitize.py).  Reads one call per line from stdin and
// prints its status:
//   op x r w s M H dtype norm mode write_y q bs y
//   quant y s M H dtype mode q bs
//   gemm mx a sa as b sb bs M N K out
//   gemm4 a sa ags b sb bgs M N K out
//   traffic nsrc ndst rows threads grid flags src0 src1 srb0 srb1 dst0..dst3 drb0..drb3
//   probe kind in n param out
//   fdec x r ro w s M H dtype write_y q y b bs N out
//   bsb M H                       (prints nq_block_scale_bytes)
// Addresses and sizes are decimal 64-bit integers; param is a decimal float.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "gnq_validate.hpp"

using namespace gnq;

static const void *P(uint64_t v) { return (const void *)(uintptr_t)v; }

int main() {
  char line[4096];
  while (std::fgets(line, sizeof line, stdin)) {
    char cmd[16];
    int off = 0;
    if (std::sscanf(line, "%15s%n", cmd, &off) != 1) continue;
    const char *p = line + off;
    auto next = [&](uint64_t &v) {
      int n = 0;
      if (std::sscanf(p, " %" SCNu64 "%n", &v, &n) != 1) std::abort();
      p += n;
    };
    auto nexti = [&](int64_t &v) {
      int n = 0;
      if (std::sscanf(p, " %" SCNd64 "%n", &v, &n) != 1) std::abort();
      p += n;
    };
    const std::string c = cmd;
    if (c == "op") {
      uint64_t x, r, w, s, q, bs, y;
      int64_t M, H, dt, norm, mode, wy;
      next(x), next(r), next(w), next(s), nexti(M), nexti(H), nexti(dt), nexti(norm), nexti(mode), nexti(wy);
      next(q), next(bs), next(y);
      std::printf("%d\n", (int)check_op(P(x), P(r), P(w), (const float *)P(s), M, H, (int)dt, (int)norm,
                                        (int)mode, (int)wy, P(q), P(bs), P(y)));
    } else if (c == "quant") {
      uint64_t y, s, q, bs;
      int64_t M, H, dt, mode;
      next(y), next(s), nexti(M), nexti(H), nexti(dt), nexti(mode), next(q), next(bs);
      std::printf("%d\n", (int)check_quant(P(y), (const float *)P(s), M, H, (int)dt, (int)mode, P(q), P(bs)));
    } else if (c == "gemm") {
      uint64_t a, sa, as, b, sb, bs, out;
      int64_t mx, M, N, K;
      nexti(mx), next(a), next(sa), next(as), next(b), next(sb), next(bs), nexti(M), nexti(N), nexti(K), next(out);
      std::printf("%d\n", (int)check_gemm_fp8(mx != 0, P(a), P(sa), (const float *)P(as), P(b), P(sb),
                                              (const float *)P(bs), M, N, K, P(out)));
    } else if (c == "gemm4") {
      uint64_t a, sa, ags, b, sb, bgs, out;
      int64_t M, N, K;
      next(a), next(sa), next(ags), next(b), next(sb), next(bgs), nexti(M), nexti(N), nexti(K), next(out);
      std::printf("%d\n", (int)check_gemm_nvfp4(P(a), P(sa), (const float *)P(ags), P(b), P(sb),
                                                (const float *)P(bgs), M, N, K, P(out)));
    } else if (c == "traffic") {
      int64_t nsrc, ndst, rows, threads, grid, flags;
      nexti(nsrc), nexti(ndst), nexti(rows), nexti(threads), nexti(grid), nexti(flags);
      uint64_t src[2], dst[4];
      int64_t srb[2], drb[4];
      next(src[0]), next(src[1]), nexti(srb[0]), nexti(srb[1]);
      for (int i = 0; i < 4; ++i) next(dst[i]);
      for (int i = 0; i < 4; ++i) nexti(drb[i]);
      const void *sp[2] = {P(src[0]), P(src[1])};
      void *dp[4] = {(void *)P(dst[0]), (void *)P(dst[1]), (void *)P(dst[2]), (void *)P(dst[3])};
      // the counts index these fixed arrays only after the check bounds them
      std::printf("%d\n", (int)check_traffic(sp, srb, (int)nsrc, dp, drb, (int)ndst, rows, (int)threads,
                                             (int)grid, (int)flags));
    } else if (c == "probe") {
      int64_t kind, n;
      uint64_t in, out;
      float param;
      int k = 0;
      nexti(kind), next(in), nexti(n);
      if (std::sscanf(p, " %f%n", &param, &k) != 1) std::abort();
      p += k;
      next(out);
      std::printf("%d\n", (int)check_convert_probe((int)kind, P(in), n, param, P(out)));
    } else if (c == "fdec") {
      uint64_t x, r, ro, w, s, q, y, b, bs, out;
      int64_t M, H, dt, wy, N;
      next(x), next(r), next(ro), next(w), next(s), nexti(M), nexti(H), nexti(dt), nexti(wy), next(q), next(y);
      next(b), next(bs), nexti(N), next(out);
      std::printf("%d\n", (int)check_fused_decode(P(x), P(r), P(ro), P(w), (const float *)P(s), M, H, (int)dt,
                                                  (int)wy, P(q), P(y), P(b), (const float *)P(bs), N, P(out)));
    } else if (c == "bsb") {
      int64_t M, H;
      nexti(M), nexti(H);
      std::printf("%zu\n", block_scale_bytes(M, H));
    } else {
      std::abort();
    }
  }
  return 0;
}
