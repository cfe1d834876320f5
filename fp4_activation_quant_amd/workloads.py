"""Seeded synthetic workloads for the fused add + Gemma RMSNorm + quant op.

This module only draws inputs: it holds none of the op's arithmetic.  Tests,
the benchmark and the smoke check all take their inputs from here, so every
side sees the same tensors.  The per-workload quant scales depend on the
op's output (amax of the normed activation); they are not computed here but
read from ``tests/golden/workload_scales.json``, which a committed script
writes from the CPU oracle.

Recipe (all draws are fp32 on the CPU from ``torch.Generator().manual_seed``,
scaled, then rounded to the activation dtype):

* seeds: ``seed_base + stream``; stream 0 = x, 1 = residual, 2 = weight,
  3 = outlier mask; the calibration draw of the decode sweep uses streams
  10, 11 and 13 for x, residual and mask (same weight).
* ``N(0, s)`` takes s as the standard deviation.
* element outliers: elements with ``rand < p`` are multiplied by f before
  rounding (x only); row outliers: rows with ``rand < p`` are multiplied by f
  in both x and residual (row M//2 if the draw picks none).
"""

from dataclasses import dataclass, field
import json
import os

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCALES_JSON = os.path.join(ROOT, "tests", "golden", "workload_scales.json")

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    H: int
    dtype: str            # "bf16" | "fp16"
    mode: str             # "fp8" (static) | "nvfp4" | "mxfp8"
    has_residual: bool
    write_y: bool
    eps: float
    x_std: float
    r_std: float
    w_dist: tuple         # ("normal", std) | ("uniform", lo, hi)
    seed_base: int
    scale_rule: str       # "fixed" | "fp8_amax" | "fp8_amax_calibration" | "nvfp4_amax" | "none"
    fixed_scale: float = 0.0
    elem_outliers: tuple = ()   # (p, factor) on x elements
    row_outliers: tuple = ()    # (p, factor) on rows of x and residual
    draw_M: int = 0             # rows drawn (>= M); 0 means M
    tags: tuple = field(default=())

    @property
    def nvfp4(self):
        return self.mode == "nvfp4"

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def rows_drawn(self):
        return self.draw_M or self.M


def _wl(**kw):
    return Workload(**kw)


_DECODE = dict(H=4096, dtype="bf16", mode="fp8", has_residual=True, write_y=False, eps=1e-6,
               x_std=1.0, r_std=2.0, w_dist=("normal", 0.1), seed_base=2000,
               scale_rule="fp8_amax_calibration", elem_outliers=(0.01, 20.0), draw_M=256)
_WIDE = dict(M=4096, H=5120, dtype="fp16", write_y=False, eps=1e-5, x_std=0.5, r_std=4.0,
             w_dist=("uniform", -0.5, 0.5), seed_base=4000, row_outliers=(0.001, 100.0))

WORKLOADS = {w.name: w for w in [
    _wl(name="fp8_m16_h2048_bf16_y", M=16, H=2048, dtype="bf16", mode="fp8", has_residual=True,
        write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1), seed_base=1000,
        scale_rule="fixed", fixed_scale=0.05),
    *[_wl(name=f"fp8_decode_m{m}_h4096_bf16", M=m, **_DECODE) for m in (1, 8, 64, 256)],
    _wl(name="nvfp4_prefill_m8192_h4096_bf16_y", M=8192, H=4096, dtype="bf16", mode="nvfp4",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=3000, scale_rule="nvfp4_amax"),
    _wl(name="fp8_res_m4096_h5120_fp16", mode="fp8", has_residual=True, scale_rule="fp8_amax", **_WIDE),
    _wl(name="fp8_nores_m4096_h5120_fp16", mode="fp8", has_residual=False, scale_rule="fp8_amax", **_WIDE),
    _wl(name="nvfp4_res_m4096_h5120_fp16", mode="nvfp4", has_residual=True, scale_rule="nvfp4_amax", **_WIDE),
    _wl(name="nvfp4_nores_m4096_h5120_fp16", mode="nvfp4", has_residual=False, scale_rule="nvfp4_amax", **_WIDE),
    _wl(name="nvfp4_m32768_h8192_bf16_y", M=32768, H=8192, dtype="bf16", mode="nvfp4",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=5000, scale_rule="nvfp4_amax"),
    # Static FP8 at the prefill and the largest shape (bf16, residual, y
    # written): the FP8 mode at sizes where bandwidth, not launch latency,
    # sets the time.
    _wl(name="fp8_prefill_m8192_h4096_bf16_y", M=8192, H=4096, dtype="bf16", mode="fp8",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=3100, scale_rule="fp8_amax"),
    _wl(name="fp8_m32768_h8192_bf16_y", M=32768, H=8192, dtype="bf16", mode="fp8",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=5100, scale_rule="fp8_amax"),
    # MXFP8 output (scales from the data, no scale argument) at the prefill
    # and the largest shape.
    _wl(name="mxfp8_prefill_m8192_h4096_bf16_y", M=8192, H=4096, dtype="bf16", mode="mxfp8",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=6000, scale_rule="none"),
    _wl(name="mxfp8_m32768_h8192_bf16_y", M=32768, H=8192, dtype="bf16", mode="mxfp8",
        has_residual=True, write_y=True, eps=1e-6, x_std=1.0, r_std=1.0, w_dist=("normal", 0.1),
        seed_base=7000, scale_rule="none"),
]}

# The workload bench.py times by default: the largest one, bandwidth-bound.
DEFAULT_BENCH = "nvfp4_m32768_h8192_bf16_y"


def _gen(seed):
    return torch.Generator().manual_seed(seed)


def _draw(wl: Workload, rows: int, x_stream: int, r_stream: int, mask_stream: int):
    H, dt = wl.H, wl.torch_dtype
    x = torch.randn(rows, H, generator=_gen(wl.seed_base + x_stream)) * wl.x_std
    r = torch.randn(rows, H, generator=_gen(wl.seed_base + r_stream)) * wl.r_std if wl.has_residual else None
    if wl.elem_outliers:
        p, f = wl.elem_outliers
        mask = torch.rand(rows, H, generator=_gen(wl.seed_base + mask_stream)) < p
        x = torch.where(mask, x * f, x)
    if wl.row_outliers:
        p, f = wl.row_outliers
        rmask = torch.rand(rows, generator=_gen(wl.seed_base + mask_stream)) < p
        if not bool(rmask.any()):
            rmask[rows // 2] = True
        x = torch.where(rmask[:, None], x * f, x)
        if r is not None:
            r = torch.where(rmask[:, None], r * f, r)
    return x.to(dt), (r.to(dt) if r is not None else None)


def make_weight(wl: Workload) -> torch.Tensor:
    g = _gen(wl.seed_base + 2)
    if wl.w_dist[0] == "normal":
        w = torch.randn(wl.H, generator=g) * wl.w_dist[1]
    else:
        lo, hi = wl.w_dist[1], wl.w_dist[2]
        w = torch.rand(wl.H, generator=g) * (hi - lo) + lo
    return w.to(wl.torch_dtype)


def make_inputs(wl: Workload):
    """(x, residual or None, weight) as CPU tensors of the workload's dtype."""
    x, r = _draw(wl, wl.rows_drawn, 0, 1, 3)
    if wl.rows_drawn != wl.M:
        x = x[: wl.M].contiguous()
        r = r[: wl.M].contiguous() if r is not None else None
    return x, r, make_weight(wl)


def make_calibration_inputs(wl: Workload):
    """The separate calibration draw of the decode sweep (same weight)."""
    x, r = _draw(wl, wl.rows_drawn, 10, 11, 13)
    return x, r, make_weight(wl)


def load_scale(wl: Workload) -> float:
    """The workload's fp32 quant scale: fixed, or read from the stored table
    (1.0, unused, for MXFP8)."""
    if wl.scale_rule == "none":
        return 1.0
    if wl.scale_rule == "fixed":
        return float(torch.tensor(wl.fixed_scale, dtype=torch.float32))
    with open(SCALES_JSON) as f:
        table = json.load(f)
    return float.fromhex(table[wl.name]["scale_hex"])


# ---------------------------------------------------------------------------
# Consumer-GEMM workloads: the quantized activation of a norm workload's
# shape (M tokens x K = H) against an (N, K) weight in the same format.
# Codes are drawn directly as bytes (no quantization arithmetic here): sign
# and mantissa uniform, E4M3 exponent field uniform in [lo, hi] (never the
# NaN pattern); E8M0 block scales uniform in [s_lo, s_hi].

@dataclass(frozen=True)
class GemmWorkload:
    name: str
    mode: str             # "mxfp8" | "fp8" | "nvfp4"
    M: int
    N: int
    K: int
    seed_base: int
    exp_range: tuple = (3, 11)          # activation codes: |v| in [2^-4, 2^4]
    w_exp_range: tuple = (0, 7)         # weight codes: |v| below 2^1
    scale_range: tuple = (118, 126)     # E8M0 codes of both operands
    a_scale: float = 0.02               # static FP8 tensor scales
    b_scale: float = 0.004
    fp4_scale_range: tuple = (0x30, 0x60)   # NVFP4 E4M3 block-scale codes (0.5 .. 32)
    a_gs: float = 300.0                 # NVFP4 global scales
    b_gs: float = 150.0


GEMM_WORKLOADS = {g.name: g for g in [
    GemmWorkload("gemm_mxfp8_m8192_n4096_k4096", "mxfp8", 8192, 4096, 4096, 8000),
    GemmWorkload("gemm_fp8_m8192_n4096_k4096", "fp8", 8192, 4096, 4096, 8100),
    GemmWorkload("gemm_mxfp8_m32768_n8192_k8192", "mxfp8", 32768, 8192, 8192, 8200),
    GemmWorkload("gemm_fp8_m32768_n8192_k8192", "fp8", 32768, 8192, 8192, 8500),
    GemmWorkload("gemm_mxfp8_m256_n4096_k4096", "mxfp8", 256, 4096, 4096, 8300),
    GemmWorkload("gemm_mxfp8_m64_n4096_k4096", "mxfp8", 64, 4096, 4096, 8400),
    GemmWorkload("gemm_mxfp8_m1_n4096_k4096", "mxfp8", 1, 4096, 4096, 8600),
    GemmWorkload("gemm_fp8_m64_n4096_k4096", "fp8", 64, 4096, 4096, 8700),
    GemmWorkload("gemm_mxfp8_m512_n4096_k4096", "mxfp8", 512, 4096, 4096, 9300),
    GemmWorkload("gemm_mxfp8_m1024_n4096_k4096", "mxfp8", 1024, 4096, 4096, 9400),
    GemmWorkload("gemm_fp8_m1024_n4096_k4096", "fp8", 1024, 4096, 4096, 9500),
    GemmWorkload("gemm_nvfp4_m8192_n4096_k4096", "nvfp4", 8192, 4096, 4096, 8800),
    GemmWorkload("gemm_nvfp4_m64_n4096_k4096", "nvfp4", 64, 4096, 4096, 8900),
    GemmWorkload("gemm_nvfp4_m1_n4096_k4096", "nvfp4", 1, 4096, 4096, 9000),
    GemmWorkload("gemm_nvfp4_m256_n4096_k4096", "nvfp4", 256, 4096, 4096, 9100),
    GemmWorkload("gemm_nvfp4_m1024_n4096_k4096", "nvfp4", 1024, 4096, 4096, 9200),
]}


def _draw_codes(rows, cols, exp_range, gen):
    lo, hi = exp_range
    sign = torch.randint(0, 2, (rows, cols), generator=gen, dtype=torch.int32) << 7
    ex = torch.randint(lo, hi + 1, (rows, cols), generator=gen, dtype=torch.int32)
    man = torch.randint(0, 8, (rows, cols), generator=gen, dtype=torch.int32)
    man = torch.where((ex == 15) & (man == 7), man - 1, man)        # no NaN code
    return (sign | (ex << 3) | man).to(torch.uint8)


def _nvfp4_scale_buffer(rows, K, code_range, gen):
    """A 128x4-tiled block-scale buffer (round_up(rows, 128) x K/16 bytes, the
    op's layout) filled with E4M3 codes in code_range (padding rows too)."""
    lo, hi = code_range
    n = (rows + 127) // 128 * 128 * (K // 16)
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int32).to(torch.uint8)


def make_gemm_inputs(gw: GemmWorkload):
    """(a codes, a scales or None, b codes, b scales or None) as CPU uint8
    tensors: FP8 codes (rows, K) with E8M0 scales (rows, K/32) for MXFP8;
    for NVFP4 packed random E2M1 codes (rows, K/2) with flat 128x4-tiled
    E4M3 scale buffers."""
    if gw.mode == "nvfp4":
        a = torch.randint(0, 256, (gw.M, gw.K // 2), generator=_gen(gw.seed_base), dtype=torch.int32)
        b = torch.randint(0, 256, (gw.N, gw.K // 2), generator=_gen(gw.seed_base + 1), dtype=torch.int32)
        sa = _nvfp4_scale_buffer(gw.M, gw.K, gw.fp4_scale_range, _gen(gw.seed_base + 2))
        sb = _nvfp4_scale_buffer(gw.N, gw.K, gw.fp4_scale_range, _gen(gw.seed_base + 3))
        return a.to(torch.uint8), sa, b.to(torch.uint8), sb
    a = _draw_codes(gw.M, gw.K, gw.exp_range, _gen(gw.seed_base))
    b = _draw_codes(gw.N, gw.K, gw.w_exp_range, _gen(gw.seed_base + 1))
    if gw.mode != "mxfp8":
        return a, None, b, None
    lo, hi = gw.scale_range
    sa = torch.randint(lo, hi + 1, (gw.M, gw.K // 32), generator=_gen(gw.seed_base + 2), dtype=torch.int32)
    sb = torch.randint(lo, hi + 1, (gw.N, gw.K // 32), generator=_gen(gw.seed_base + 3), dtype=torch.int32)
    return a, sa.to(torch.uint8), b, sb.to(torch.uint8)
