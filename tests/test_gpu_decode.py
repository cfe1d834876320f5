"""The fused decode step (nq_gemma_add_rms_norm_quant_gemm_fp8: the op in
static FP8 mode on a few rows and its consumer linear; one launch up to 3
rows, the op and the decode GEMM from 4) against the two calls it replaces,
through the C ABI:

  * the op's outputs (x + residual, FP8 codes, y) bit-for-bit those of
    nq_gemma_add_rms_norm_quant (which the parity tests check against the
    oracle);
  * the linear's bf16 output bit-for-bit that of nq_gemm_fp8_static on the
    same codes from 4 rows, and up to 3 rows where that call runs the
    decode GEMM on 32 x 16 tiles (K 2048 or 4096, N < 6144: the same K
    split, MFMA sequence and reduction order), and everywhere within the
    GEMM bar against the oracle's exact product
    (|out - exact| <= 2^-8 |exact| + 2^-10 sum |a b|);
  * x and residual unchanged; nothing written past any output."""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib, ops
from tests import parity as P
from tests.test_gpu_gemm import _finite_codes, _tolerance_check

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _guarded(shape, dtype, dev):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((n + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device=dev)
    return buf, buf[:n].view(dtype).view(*shape)


CASES = [
    # dtype, M, H, N, residual, write_y
    (torch.bfloat16, 1, 4096, 4096, True, False),
    (torch.bfloat16, 2, 4096, 4096, True, True),
    (torch.bfloat16, 3, 4096, 1000, True, False),
    (torch.bfloat16, 3, 2048, 4096, True, True),     # the largest one-launch case, 4-row kernel
    (torch.float16, 3, 1024, 4100, False, True),
    (torch.bfloat16, 4, 4096, 4096, False, True),
    (torch.bfloat16, 8, 4096, 4096, True, True),
    (torch.float16, 5, 2048, 4096, True, False),
    (torch.bfloat16, 8, 2048, 2048, True, True),
    (torch.float16, 7, 4096, 17, True, True),        # one partial workgroup of weight rows + one more
    (torch.bfloat16, 6, 4096, 8192, True, False),    # the two-call GEMM takes 32 x 32 tiles here
    (torch.bfloat16, 1, 1024, 512, True, True),      # K = 1024: the two-call GEMM is the skinny kernel
    (torch.float16, 8, 1024, 300, False, False),
]


@pytest.mark.parametrize("dt,M,H,N,res,wy", CASES)
def test_fused_decode_matches_the_two_calls(dt, M, H, N, res, wy):
    print(f"fused decode {dt} M={M} H={H} N={N} res={res} write_y={wy}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M * 131 + H + N)
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt) if res else None
    w = (torch.randn(H, generator=g) * 0.1).to(dt)
    s = torch.tensor([0.02], dtype=torch.float32, device=dev)
    rng = np.random.default_rng(M + H + N)
    bq = rng.integers(0, 8, size=(N, H), dtype=np.int64) | (rng.integers(0, 8, size=(N, H)) << 3) \
        | (rng.integers(0, 2, size=(N, H)) << 7)                       # |v| < 2, no NaN code
    bq = bq.astype(np.uint8)
    bd = torch.from_numpy(bq).to(dev)
    bs = torch.tensor([0.004], dtype=torch.float32, device=dev)
    xd, wd = x.to(dev), w.to(dev)
    rd = r.to(dev) if res else None

    rbuf, rout = _guarded((M, H), dt, dev) if res else (None, None)
    qbuf, q = _guarded((M, H), torch.uint8, dev)
    ybuf, y = _guarded((M, H), dt, dev) if wy else (None, None)
    obuf, out = _guarded((M, N), torch.bfloat16, dev)
    ops.gemma_add_rms_norm_quant_gemm_fp8_out(xd, rd, rout, wd, 1e-6, s, bd, bs, q, y, out)
    torch.cuda.synchronize()
    for buf, t in ((rbuf, rout), (qbuf, q), (ybuf, y), (obuf, out)):
        if buf is not None:
            n = t.numel() * t.element_size()
            assert bool((buf[n:] == P.SENTINEL).all()), "wrote past an output"
    assert torch.equal(xd.cpu(), x)
    if res:
        assert torch.equal(rd.cpu(), r)                                # read only

    # the two calls
    r2 = rd.clone() if res else None
    q2 = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
    y2 = torch.empty((M, H), dtype=dt, device=dev) if wy else None
    ops.gemma_add_rms_norm_quant_out(xd, r2, wd, 1e-6, s, False, q2, None, y2)
    out2 = ops.gemm_fp8_static(q2.view(torch.uint8), s, bd, bs)
    torch.cuda.synchronize()
    if res:
        assert torch.equal(rout.cpu(), r2.cpu())
    assert torch.equal(q.cpu(), q2.view(torch.uint8).cpu())
    if wy:
        assert torch.equal(y.cpu(), y2.cpu())
    got = P.bits16(out)
    if M >= 4 or (H in (2048, 4096) and N < 6144):
        assert np.array_equal(got, P.bits16(out2))
    else:
        print(f"  output equal to the two-call GEMM: {np.array_equal(got, P.bits16(out2))}", flush=True)
    aq = q.cpu().numpy()
    exact, _ = O.gemm_fp8_static(aq, 0.02, bq, 0.004)
    mag = O.gemm_f64(np.abs(O.dequant_fp8_static(aq, 0.02)), np.abs(O.dequant_fp8_static(bq, 0.004)))
    _tolerance_check(got, exact, mag)


def test_fused_decode_rejects_and_passes_through():
    dev = torch.device("cuda")
    x = torch.randn(2, 4096, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(4096, dtype=torch.bfloat16, device=dev)
    s = torch.ones(1, dtype=torch.float32, device=dev)
    b = torch.zeros(64, 4096, dtype=torch.uint8, device=dev)
    q = torch.empty(2, 4096, dtype=torch.uint8, device=dev)
    out = torch.empty(2, 64, dtype=torch.bfloat16, device=dev)
    r = torch.randn(2, 4096, dtype=torch.bfloat16, device=dev)
    with pytest.raises(_lib.NqError) as e:          # in place: residual_out is residual
        ops.gemma_add_rms_norm_quant_gemm_fp8_out(x, r, r, w, 1e-6, s, b, s, q, None, out)
    assert e.value.status == _lib.NQ_EINVAL
    x9 = torch.randn(9, 4096, dtype=torch.bfloat16, device=dev)
    with pytest.raises(_lib.NqError) as e:          # more than 8 rows: two calls instead
        ops.gemma_add_rms_norm_quant_gemm_fp8_out(x9, None, None, w, 1e-6, s, b, s,
                                                  torch.empty(9, 4096, dtype=torch.uint8, device=dev), None,
                                                  torch.empty(9, 64, dtype=torch.bfloat16, device=dev))
    assert e.value.status == _lib.NQ_EUNSUPPORTED


@pytest.mark.parametrize("M,H", [(1, 4096), (3, 2048), (5, 1024)])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_fused_decode_zero_products_keep_their_sign(M, H, dt):
    """Columns with w = -1 (Gemma's 1 + w is +0) and half a row with x =
    -residual (h = +0): y is a zero product with the product's sign, and the decode
    step's codes and y must equal the separate op's, sign of zero included
    (which the op's own tests check against the oracle)."""
    print(f"fused decode zero products M={M} H={H} {dt}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M * 7 + H)
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt)
    r[0, : H // 2] = -x[0, : H // 2]
    w = (torch.randn(H, generator=g) * 0.1).to(dt)
    w[::7] = -1.0
    s = torch.tensor([0.02], dtype=torch.float32, device=dev)
    N = 256
    rng = np.random.default_rng(M + H)
    bq = torch.from_numpy(_finite_codes(rng, (N, H))).to(dev)
    bs = torch.tensor([0.004], dtype=torch.float32, device=dev)
    xd, wd, rd = x.to(dev), w.to(dev), r.to(dev)
    rout = torch.empty_like(rd)
    q = torch.empty((M, H), dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=dt, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ops.gemma_add_rms_norm_quant_gemm_fp8_out(xd, rd, rout, wd, 1e-6, s, bq, bs, q, y, out)
    r2 = rd.clone()
    q2 = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
    y2 = torch.empty((M, H), dtype=dt, device=dev)
    ops.gemma_add_rms_norm_quant_out(xd, r2, wd, 1e-6, s, False, q2, None, y2)
    torch.cuda.synchronize()
    assert torch.equal(rout.cpu().view(torch.int16), r2.cpu().view(torch.int16))
    assert torch.equal(y.cpu().view(torch.int16), y2.cpu().view(torch.int16))
    assert torch.equal(q.cpu(), q2.view(torch.uint8).cpu())
    yb = P.bits16(y)
    assert np.count_nonzero(yb == 0x8000) > 0 and np.count_nonzero(yb == 0x0000) > 0
