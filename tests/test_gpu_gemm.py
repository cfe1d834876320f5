"""GPU parity of the consumer GEMM (nq_gemm_mxfp8, nq_gemm_fp8_static)
against the oracle, through the C ABI.

Bars:
  * exact cases -- operands whose products and partial sums are exact in any
    accumulator (a few significant bits, moderate scales): the bf16 output is
    bit-identical to the oracle's rounding of the exact sum.  These pin the
    operand layout, the K pairing and the per-block scales;
  * general random codes and scales: |out - exact| <= 2^-8 |exact| (bf16
    rounding of the accumulator) + 2^-10 * sum_k |a_k b_k| (the block-scaled
    MFMA sums its 64 products with a relative error measured up to ~2^-12.8
    of their absolute sum; fp32 accumulation across steps adds far less).
Output guard bytes after the (M, N) result must keep their sentinel.
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib, ops
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


# E4M3 codes of small exact values: 0, +-0.5, +-1, +-1.5, +-2, +-3, +-4
_SMALL = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48,
                   0xB0, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8], np.uint8)


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    return np.where((c & 0x7F) == 0x7F, c - 1, c).astype(np.uint8)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(mx, aq, as_, bq, bs, M, N):
    """GPU result as bf16 bits, with a guarded output buffer."""
    out = torch.full((M * N * 2 + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device="cuda")
    o = out[:M * N * 2].view(torch.bfloat16).view(M, N)
    if mx:
        ops.gemm_mxfp8(_dev(aq), _dev(as_), _dev(bq), _dev(bs), out=o)
    else:
        ops.gemm_fp8_static(_dev(aq), torch.tensor([as_], dtype=torch.float32, device="cuda"),
                            _dev(bq), torch.tensor([bs], dtype=torch.float32, device="cuda"), out=o)
    torch.cuda.synchronize()
    assert bool((out[M * N * 2:] == P.SENTINEL).all()), "wrote past the output"
    return P.bits16(o)


# kernels: M <= 256 with K % 2048 == 0 and K <= 16384 -> decode kernel;
# other M <= 256 with K % 64 == 0 -> skinny; K % 512 == 0 -> LDS-DMA
# pipeline; otherwise the register-staged kernel.  (2000, 300, 1024) and
# (1030, 1800, 512) have a multiple of 8 output tiles (the per-XCD tile
# renumbering) with ragged edges; K = 512 is a single chunk of 8 steps.
# The decode shapes cover each of its tiles (64 x 64 when those number
# >= 256 and K <= 8192, else 32 x 16 when 32 x 32 tiles would number fewer
# than 192, else 32 x 32) with ragged edges, and K from 2048 (four stages
# per wave) to 16384 (the largest scale slab).
SHAPES = [(1, 8, 64), (5, 300, 96), (256, 256, 128), (300, 520, 1056), (513, 257, 2048),
          (64, 1024, 4096), (1000, 40, 160), (300, 600, 4096), (257, 1100, 1536),
          (2000, 300, 1024), (1030, 1800, 512),
          (1, 4096, 2048), (33, 300, 2048), (7, 1000, 6144), (250, 130, 8192), (3, 64, 16384),
          (20, 200, 2048), (9, 50, 4096), (70, 2100, 2048), (200, 5000, 2048),
          (2100, 4096, 512), (200, 16384, 512)]
# Tile paths: K % 512 != 0 beyond 256 rows -> register-staged 256 x 256
# kernel ((300, 520, 1056), (1000, 40, 160)); (2100, 4096) -> 144 workgroups
# of 256 x 256; the other M > 256 shapes and (200, 16384) -> 128 x 128;
# M <= 256 otherwise -> decode or skinny kernels.


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_mxfp8_gemm_exact_cases(M, N, K):
    print(f"gemm mx exact M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 7 + N * 11 + K)
    aq = _SMALL[rng.integers(0, len(_SMALL), size=(M, K))]
    bq = _SMALL[rng.integers(0, len(_SMALL), size=(N, K))]
    # block scales 2^-1 .. 2^1: every product is a multiple of 2^-4 below 64,
    # so all sums up to K = 4096 stay within 22 bits (exact in fp32)
    as_ = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
    bs = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    got = _run(True, aq, as_, bq, bs, M, N)
    _, want = O.gemm_mxfp8(aq, as_, bq, bs)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], want[bad][:5])


@pytest.mark.parametrize("M,N,K", SHAPES[:5] + SHAPES[7:])
def test_fp8_static_gemm_exact_cases(M, N, K):
    print(f"gemm static exact M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 5 + N * 3 + K)
    aq = _SMALL[rng.integers(0, len(_SMALL), size=(M, K))]
    bq = _SMALL[rng.integers(0, len(_SMALL), size=(N, K))]
    got = _run(False, aq, 0.25, bq, 2.0, M, N)
    _, want = O.gemm_fp8_static(aq, 0.25, bq, 2.0)
    assert np.array_equal(got, want)


def _tolerance_check(got_bits, exact, mag):
    got = O.bits_to_f64(got_bits, O.BF16)
    tol = 2.0 ** -8 * np.abs(exact) + 2.0 ** -10 * mag + 1e-300
    err = np.abs(got - exact)
    worst = float(np.max(err / tol))
    print(f"  worst err / tol = {worst:.3f}", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("M,N,K", [(37, 300, 512), (256, 512, 4096), (129, 130, 1056), (512, 384, 4096),
                                   (300, 260, 160), (17, 96, 16384), (1, 333, 4096), (100, 2000, 4096),
                                   (250, 4100, 4096), (2100, 4096, 1024), (1030, 1800, 1024)])
def test_mxfp8_gemm_random(M, N, K):
    print(f"gemm mx random M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    aq, bq = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    as_ = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    bs = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    got = _run(True, aq, as_, bq, bs, M, N)
    exact, _ = O.gemm_mxfp8(aq, as_, bq, bs)
    mag = O.gemm_f64(np.abs(O.dequant_mxfp8(aq, as_)), np.abs(O.dequant_mxfp8(bq, bs)))
    _tolerance_check(got, exact, mag)


@pytest.mark.parametrize("M,N,K", [(200, 300, 2048), (600, 300, 2048), (2100, 4096, 512), (200, 16384, 512)])
def test_fp8_static_gemm_random(M, N, K):
    rng = np.random.default_rng(17)
    aq, bq = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    got = _run(False, aq, 0.0137, bq, 0.0021, M, N)
    exact, _ = O.gemm_fp8_static(aq, 0.0137, bq, 0.0021)
    mag = O.gemm_f64(np.abs(O.dequant_fp8_static(aq, 0.0137)), np.abs(O.dequant_fp8_static(bq, 0.0021)))
    _tolerance_check(got, exact, mag)


@pytest.mark.parametrize("mode", ["mxfp8", "fp8"])
def test_gemm_consumes_the_ops_quantized_output(mode):
    """The op's codes and scales go straight into the consumer linear.  The
    oracle computes the op's codes from the seeded inputs and the GEMM of
    those codes; on the GPU the op's own output feeds the GEMM.  Rows whose
    GPU codes equal the oracle's (all but a few: y may differ by one unit
    near a rounding tie) must match the oracle GEMM within the tolerance."""
    print(f"gemm consumer {mode}", flush=True)
    g = torch.Generator().manual_seed(23)
    M, H, N = 300, 4096, 384
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    r = torch.randn(M, H, generator=g).to(torch.bfloat16)
    w = (torch.randn(H, generator=g) * 0.1).to(torch.bfloat16)
    rng = np.random.default_rng(3)
    wq = _finite_codes(rng, (N, H))
    wq = np.where((wq & 0x78) > 0x50, wq & 0x87, wq).astype(np.uint8)   # keep |w| <= 16
    xd, rd, wd = x.cuda(), r.cuda(), w.cuda()
    if mode == "mxfp8":
        ws = rng.integers(118, 124, size=(N, H // 32)).astype(np.uint8)
        ref = O.add_rms_norm_quant(P.bits16(x), P.bits16(r), P.bits16(w), 1e-6, 1.0, "mxfp8")
        exact, _ = O.gemm_mxfp8(ref["q"], ref["scales"], wq, ws)
        mag = O.gemm_f64(np.abs(O.dequant_mxfp8(ref["q"], ref["scales"])), np.abs(O.dequant_mxfp8(wq, ws)))
        q, s, _ = ops.add_rms_norm_quant(xd, rd, wd, 1e-6, None, "mxfp8")
        out = ops.gemm_mxfp8(q, s, _dev(wq), _dev(ws))
        same = np.all(q.view(torch.uint8).cpu().numpy() == ref["q"], axis=1) & \
            np.all(s.view(torch.uint8).cpu().numpy() == ref["scales"], axis=1)
    else:
        ref = O.add_rms_norm_quant(P.bits16(x), P.bits16(r), P.bits16(w), 1e-6, 0.02, "fp8")
        exact, _ = O.gemm_fp8_static(ref["q"], 0.02, wq, 0.004)
        mag = O.gemm_f64(np.abs(O.dequant_fp8_static(ref["q"], 0.02)), np.abs(O.dequant_fp8_static(wq, 0.004)))
        sa = torch.tensor([0.02], dtype=torch.float32, device="cuda")
        sw = torch.tensor([0.004], dtype=torch.float32, device="cuda")
        q, _, _ = ops.gemma_add_rms_norm_quant(xd, rd, wd, 1e-6, sa, False)
        out = ops.gemm_fp8_static(q, sa, _dev(wq), sw)
        same = np.all(q.view(torch.uint8).cpu().numpy() == ref["q"], axis=1)
    torch.cuda.synchronize()
    print(f"  rows with the oracle's codes: {int(same.sum())} / {M}", flush=True)
    assert same.mean() >= 0.95
    _tolerance_check(P.bits16(out)[same], exact[same], mag[same])


def test_gemm_empty_writes_nothing():
    buf = torch.full((1 << 16,), P.SENTINEL, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = _lib.nq_gemm_mxfp8(p, p + 8192, p + 16384, p + 24576, 0, 64, 64, p + 32768, 0)
    st2 = _lib.nq_gemm_mxfp8(p, p + 8192, p + 16384, p + 24576, 64, 0, 64, p + 32768, 0)
    torch.cuda.synchronize()
    assert st == _lib.NQ_OK and st2 == _lib.NQ_OK and bool((buf == P.SENTINEL).all())


# ---- NVFP4 consumer (nq_gemm_nvfp4) ----------------------------------------

def _nvfp4_operand(rng, rows, K, nibbles, scale_codes):
    """Packed E2M1 codes drawn from `nibbles` and a 128x4-tiled scale buffer
    with block scales from `scale_codes`; the padding rows' bytes are random
    junk (the kernel reads them beside real rows but must not use them)."""
    nib = np.asarray(nibbles, np.uint8)[rng.integers(0, len(nibbles), size=(rows, K))]
    q = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    S = np.asarray(scale_codes, np.uint8)[rng.integers(0, len(scale_codes), size=(rows, K // 16))]
    buf = rng.integers(0, 0x7F, size=int(np.prod(O.block_scale_buffer_shape(rows, K))), dtype=np.int64).astype(np.uint8)
    O.scatter_block_scales(S, rows, K, buf)
    return q, buf


def _run_nvfp4(aq, abuf, ga, bq, bbuf, gb, M, N):
    out = torch.full((M * N * 2 + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device="cuda")
    o = out[:M * N * 2].view(torch.bfloat16).view(M, N)
    f32 = lambda v: torch.tensor([v], dtype=torch.float32, device="cuda")
    ops.gemm_nvfp4(_dev(aq), _dev(abuf), f32(ga), _dev(bq), _dev(bbuf), f32(gb), out=o)
    torch.cuda.synchronize()
    assert bool((out[M * N * 2:] == P.SENTINEL).all()), "wrote past the output"
    return P.bits16(o)


# 32 x 32 tiles up to 256 rows (8 waves when K % 512 == 0, else 4), 256 x 256
# beyond; shapes cross 128-row scale tiles and have ragged edges (a partial
# 256-row tile with and without its second 128-row group); K from 256 (one
# stage per wave; fewer stages than the large kernel's ring) up
# K % 256 != 0 included: 64-element steps split unevenly over the small
# kernel's waves (some with none) and odd step counts in the large one;
# M <= 8 with M N <= 12288 takes the dot-product kernel (each of its row
# counts 1, 2, 4, 8; (3, 4096, 256) sits on the bound), except M = 8 at
# K = 8192, whose fp16 activation exceeds its LDS; (2, 6200, 512) and
# (4, 4100, 320) lie just past the bound, on the 32 x 32 tiles; the tile
# choice puts (2100, 4096) on 256 x 256 tiles, (300, 4096) and (257, 4160)
# on 128 x 64, (200, 3072) on 64 x 64, (100, 3100) and (520, 700) on 64 x 32
# and the rest on 32 x 32.
NVFP4_SHAPES = [(1, 8, 256), (5, 300, 512), (32, 64, 1024), (33, 100, 256), (200, 130, 2048),
                (130, 257, 768), (64, 1000, 1024), (300, 200, 512), (257, 70, 768), (600, 520, 1024),
                (520, 700, 256), (1, 40, 64), (17, 96, 448), (64, 200, 1152), (260, 33, 64),
                (300, 260, 320), (257, 130, 1152), (2, 70, 320), (3, 130, 1152), (4, 17, 64),
                (8, 50, 8192), (1, 2000, 3072), (2100, 4096, 128), (300, 4096, 256), (257, 4160, 192),
                (200, 3072, 320), (100, 3100, 256), (3, 4096, 256), (2, 6200, 512), (4, 4100, 320)]


@pytest.mark.parametrize("M,N,K", NVFP4_SHAPES)
@pytest.mark.parametrize("gs", [(1.0, 1.0), (2.0, 0.5)])
def test_nvfp4_gemm_exact_cases(M, N, K, gs):
    """Codes within +-2 and block scales 0.5 .. 1.5 (non-powers of two
    included): every partial sum is a multiple of 2^-8 below 2^24 units, so
    any fp32 summation order is exact, and with power-of-two global scales
    the bf16 result is bit-identical to the oracle's rounding."""
    print(f"gemm nvfp4 exact M={M} N={N} K={K} gs={gs}", flush=True)
    rng = np.random.default_rng(M * 13 + N * 7 + K)
    nib = [0, 1, 2, 3, 4, 9, 10, 11, 12]
    sc = [0x30, 0x38, 0x39, 0x3C]
    aq, abuf = _nvfp4_operand(rng, M, K, nib, sc)
    bq, bbuf = _nvfp4_operand(rng, N, K, nib, sc)
    got = _run_nvfp4(aq, abuf, gs[0], bq, bbuf, gs[1], M, N)
    _, want = O.gemm_nvfp4(aq, abuf, gs[0], bq, bbuf, gs[1], M, N, K)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], want[bad][:5])


@pytest.mark.parametrize("M,N,K", [(17, 96, 4096), (300, 520, 2048), (1, 333, 8192), (256, 512, 4096),
                                   (300, 520, 2880), (8, 300, 2880), (2, 1000, 4096), (4, 64, 16384),
                                   (2100, 4096, 256), (300, 4096, 512), (200, 3072, 512), (100, 3100, 512)])
def test_nvfp4_gemm_random(M, N, K):
    print(f"gemm nvfp4 random M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + 3 * N + K)
    sc = [c for c in range(0x18, 0x60)]                 # E4M3 block scales 2^-4 .. 2^5
    aq, abuf = _nvfp4_operand(rng, M, K, list(range(16)), sc)
    bq, bbuf = _nvfp4_operand(rng, N, K, list(range(16)), sc)
    ga, gb = 2.7, 0.37
    got = _run_nvfp4(aq, abuf, ga, bq, bbuf, gb, M, N)
    exact, _ = O.gemm_nvfp4(aq, abuf, ga, bq, bbuf, gb, M, N, K)
    mag = O.gemm_f64(np.abs(O.dequant_nvfp4(aq, abuf, ga, M, K)), np.abs(O.dequant_nvfp4(bq, bbuf, gb, N, K)))
    _tolerance_check(got, exact, mag)


@pytest.mark.parametrize("M,H,N", [(300, 4096, 384), (40, 1152, 200)])
def test_nvfp4_gemm_consumes_the_ops_output(M, H, N):
    """The op's NVFP4 codes, block scales and global scale go straight into
    the consumer; rows whose GPU codes and scales equal the oracle's must
    match the oracle GEMM of the oracle's own output within the tolerance."""
    print(f"gemm nvfp4 consumer M={M} H={H} N={N}", flush=True)
    g = torch.Generator().manual_seed(29)
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    r = torch.randn(M, H, generator=g).to(torch.bfloat16)
    w = (torch.randn(H, generator=g) * 0.1).to(torch.bfloat16)
    gs = 448.0 * 6.0 / 9.0
    rng = np.random.default_rng(4)
    bq, bbuf = _nvfp4_operand(rng, N, H, list(range(16)), list(range(0x20, 0x48)))
    gb = 1.5
    ref = O.add_rms_norm_quant(P.bits16(x), P.bits16(r), P.bits16(w), 1e-6, gs, "nvfp4")
    abuf = np.asarray(ref["block_scale"], np.uint8).reshape(-1)
    exact, _ = O.gemm_nvfp4(ref["q"], abuf, gs, bq, bbuf, gb, M, N, H)
    mag = O.gemm_f64(np.abs(O.dequant_nvfp4(ref["q"], abuf, gs, M, H)), np.abs(O.dequant_nvfp4(bq, bbuf, gb, N, H)))
    sd = torch.tensor([gs], dtype=torch.float32, device="cuda")
    q, bs, _ = ops.gemma_add_rms_norm_quant(x.cuda(), r.cuda(), w.cuda(), 1e-6, sd, True)
    out = ops.gemm_nvfp4(q, bs, sd, _dev(bq), _dev(bbuf), torch.tensor([gb], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    qn = q.view(torch.uint8).cpu().numpy()
    bsn = bs.view(torch.uint8).cpu().numpy().reshape(-1)
    rows = np.arange(M)[:, None]
    offs = O.swizzle_128x4_offset(rows, np.arange(H // 16)[None, :], H)
    same = np.all(qn == ref["q"], axis=1) & np.all(bsn[offs] == abuf[offs], axis=1)
    print(f"  rows with the oracle's codes and scales: {int(same.sum())} / {M}", flush=True)
    assert same.mean() >= 0.95
    _tolerance_check(P.bits16(out)[same], exact[same], mag[same])


def test_nvfp4_gemm_empty_writes_nothing():
    buf = torch.full((1 << 16,), P.SENTINEL, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = _lib.nq_gemm_nvfp4(p, p + 8192, p + 16384, p + 24576, p + 32768, p + 16388, 0, 64, 256, p + 40960, 0)
    st2 = _lib.nq_gemm_nvfp4(p, p + 8192, p + 16384, p + 24576, p + 32768, p + 16388, 64, 0, 256, p + 40960, 0)
    torch.cuda.synchronize()
    assert st == _lib.NQ_OK and st2 == _lib.NQ_OK and bool((buf == P.SENTINEL).all())


def test_wrappers_reject_bad_buffers():
    """Every tensor the wrappers hand to the library by pointer is checked
    first (device, contiguity, shape / size, element type): these raise
    before anything is launched."""
    dev = torch.device("cuda")
    M, N, K = 4, 64, 256
    a = torch.zeros(M, K, dtype=torch.uint8, device=dev)
    b = torch.zeros(N, K, dtype=torch.uint8, device=dev)
    sa = torch.zeros(M, K // 32, dtype=torch.uint8, device=dev)
    sb = torch.zeros(N, K // 32, dtype=torch.uint8, device=dev)
    one = torch.ones(1, dtype=torch.float32, device=dev)
    bad_out = [torch.empty(M, N + 1, dtype=torch.bfloat16, device=dev),          # shape
               torch.empty(M, N, dtype=torch.float16, device=dev),                # dtype
               torch.empty(N, M, dtype=torch.bfloat16, device=dev).t(),          # not contiguous
               torch.empty(M, N, dtype=torch.bfloat16)]                           # host memory
    for o in bad_out:
        with pytest.raises(ValueError, match="out"):
            ops.gemm_mxfp8(a, sa, b, sb, out=o)
        with pytest.raises(ValueError, match="out"):
            ops.gemm_fp8_static(a, one, b, one, out=o)
    with pytest.raises(ValueError, match="a_scales"):
        ops.gemm_mxfp8(a, sa.cpu(), b, sb)
    with pytest.raises(ValueError, match="b_scales"):
        ops.gemm_mxfp8(a, sa, b, sb[:, :-1].contiguous())
    with pytest.raises(ValueError, match="a_scale"):
        ops.gemm_fp8_static(a, one.cpu(), b, one)
    with pytest.raises(ValueError, match="b_scale"):
        ops.gemm_fp8_static(a, one, b, torch.ones(2, dtype=torch.float32, device=dev))
    a4 = torch.zeros(M, K // 2, dtype=torch.uint8, device=dev)
    b4 = torch.zeros(N, K // 2, dtype=torch.uint8, device=dev)
    sa4 = torch.zeros(ops.block_scale_bytes(M, K), dtype=torch.uint8, device=dev)
    sb4 = torch.zeros(ops.block_scale_bytes(N, K), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="b_block_scale"):
        ops.gemm_nvfp4(a4, sa4, one, b4, sb4[:-1], one)
    with pytest.raises(ValueError, match="a_global_scale"):
        ops.gemm_nvfp4(a4, sa4, one.double(), b4, sb4, one)
    with pytest.raises(ValueError, match="out"):
        ops.gemm_nvfp4(a4, sa4, one, b4, sb4, one, out=torch.empty(M, N - 1, dtype=torch.bfloat16, device=dev))
    y = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="scale"):
        ops.quant_fp8_static(y, one.cpu())
    with pytest.raises(ValueError, match="q"):
        ops.quant_fp8_static(y, one, q=torch.empty(M, K - 1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="block_scale"):
        ops.quant_nvfp4(y, one, block_scale=torch.empty(8, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError, match="global_scale"):
        ops.quant_nvfp4(y, torch.ones(1, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError, match="scales"):
        ops.quant_mxfp8(y, scales=torch.empty(M, K // 32 + 1, dtype=torch.uint8, device=dev))


def test_op_out_forms_reject_bad_buffers():
    """The caller-buffer forms of the op check their tensors too."""
    dev = torch.device("cuda")
    M, H = 4, 256
    x = torch.zeros(M, H, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(H, dtype=torch.bfloat16, device=dev)
    s = torch.ones(1, dtype=torch.float32, device=dev)
    q = torch.empty(M, H // 2, dtype=torch.uint8, device=dev)
    bs = torch.empty(ops.block_scale_bytes(M, H), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="block_scale"):
        ops.gemma_add_rms_norm_quant_out(x, None, w, 1e-6, s, True, q, bs[:-1], None)
    with pytest.raises(ValueError, match="q"):
        ops.gemma_add_rms_norm_quant_out(x, None, w, 1e-6, s, True, q.cpu(), bs, None)
    with pytest.raises(ValueError, match="y"):
        ops.gemma_add_rms_norm_quant_out(x, None, w, 1e-6, s, True, q, bs,
                                         torch.empty(M, H, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError, match="scale"):
        ops.gemma_add_rms_norm_quant_out(x, None, w, 1e-6, s.cpu(), True, q, bs, None)
    with pytest.raises(ValueError, match="block_scale"):
        ops.add_rms_norm_quant_out(x, None, w, 1e-6, None, "mxfp8", "gemma",
                                   torch.empty(M, H, dtype=torch.uint8, device=dev),
                                   torch.empty(M, H // 32 - 1, dtype=torch.uint8, device=dev), None)
