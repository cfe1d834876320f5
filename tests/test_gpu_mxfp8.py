"""GPU parity of the MXFP8 variant (E4M3 codes, one E8M0 scale per 32-element
block, row-major), through the C ABI: the fused op at the workloads' full
sizes and on edge shapes against the oracle, the standalone MXFP8 quant bit
for bit against the oracle, the unfused chain against the fused kernel, and
the kernels' own scale and element routines (conversion probe) against the
oracle's block rule over every tie of the fp32 inputs that matter."""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib, ops
from fp4_activation_quant_amd.workloads import WORKLOADS, make_inputs
from tests import parity as P
from tests.test_gpu_convert import probe
from tests.test_oracle_formats import _tie_heavy_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _run_and_compare(x, r, w, eps, write_y, rows=None, misalign=False, norm="gemma"):
    gpu = P.run_gpu(x, r.clone() if r is not None else None, w, eps, 1.0, False, write_y,
                    misalign=misalign, norm=norm, mxfp8=True)
    y_gpu = None
    if not write_y:
        y_gpu = P.run_gpu(x, r.clone() if r is not None else None, w, eps, 1.0, False, True,
                          misalign=misalign, norm=norm, mxfp8=True)["y"]
    rows = P.all_rows(x.shape[0]) if rows is None else rows
    rep = P.compare(gpu, x, r, w, eps, 1.0, rows, y_gpu=y_gpu)
    if r is not None:
        assert np.array_equal(gpu["residual"], P.bits16(x + r))
    print(rep, flush=True)
    return P.check(rep), gpu


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if w.mode != "mxfp8"])
def test_mxfp8_workload_parity(name):
    """The other workloads' inputs and shapes with the MXFP8 output (their
    quant scale is not used: MXFP8 takes its scales from the data); the MXFP8
    workloads themselves run in the workload parity test."""
    wl = WORKLOADS[name]
    print(f"mxfp8 workload {name}", flush=True)
    x, r, w = make_inputs(wl)
    rep, _ = _run_and_compare(x, r, w, wl.eps, wl.write_y, rows=P.all_rows(wl.M))
    P.record(f"{name} (as MXFP8)", rep)


EDGE = [
    # dtype, M, H, residual, write_y
    (torch.bfloat16, 1, 32, True, True),       # one block, 4 lanes per row
    (torch.bfloat16, 300, 64, True, False),
    (torch.float16, 37, 96, False, True),      # 12 chunks -> 16 lanes per row, 4 idle
    (torch.bfloat16, 129, 160, True, True),
    (torch.bfloat16, 1000, 480, True, True),   # 60 chunks -> 64 lanes per row
    (torch.float16, 255, 512, True, False),
    (torch.bfloat16, 127, 2048, True, True),
    (torch.bfloat16, 9, 4128, True, True),     # 2 chunks per thread, ragged
    (torch.float16, 65, 5120, False, True),
    (torch.bfloat16, 3, 16384, True, True),    # 2 chunks x 1024 threads
    (torch.bfloat16, 5, 24576, True, False),   # 4 chunks per thread
    (torch.bfloat16, 3, 32768, True, True),    # 4 chunks x 1024 threads
    (torch.bfloat16, 2, 32800, True, True),    # H > 32768: scalar path
    (torch.float16, 2100, 256, True, True),
]


@pytest.mark.parametrize("dt,M,H,res,wy", EDGE)
def test_mxfp8_edge_shapes(dt, M, H, res, wy):
    print(f"mxfp8 edge {dt} M={M} H={H} res={res} write_y={wy}", flush=True)
    g = torch.Generator().manual_seed(M * 7919 + H + 1)
    # per-row magnitudes over several binades so the block scales vary (fp16
    # kept well inside its range)
    spread = 3.0 if dt == torch.bfloat16 else 1.2
    x = (torch.randn(M, H, generator=g) * torch.exp(torch.randn(M, 1, generator=g) * spread)).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt) if res else None
    w = (torch.randn(H, generator=g) * 0.2).to(dt)
    _run_and_compare(x, r, w, 1e-6, wy)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_mxfp8_unaligned_views_and_plain_norm(dt):
    print(f"mxfp8 unaligned / plain {dt}", flush=True)
    g = torch.Generator().manual_seed(7)
    M, H = 70, 256
    x = torch.randn(M, H, generator=g).to(dt)
    r = torch.randn(M, H, generator=g).to(dt)
    w = (torch.randn(H, generator=g) * 0.2 + 1).to(dt)
    _run_and_compare(x, r, w, 1e-6, True, misalign=True)
    _run_and_compare(x, r, w, 1e-6, True, norm="plain")
    _run_and_compare(x, None, w, 1e-6, False, norm="plain")


def test_mxfp8_special_values():
    """Zero rows (all-zero blocks: scale code 0), constant rows, tiny and wide
    ranges, and (1 + w) == 0 columns."""
    H = 256
    rows = [
        torch.zeros(H), torch.full((H,), 3.0), torch.full((H,), -2.0 ** -10),
        torch.linspace(-1000, 1000, H), torch.where(torch.arange(H) % 2 == 0, 1e4, -1e-3),
        torch.where(torch.arange(H) < 32, 0.0, 1.0),
    ]
    for dt in (torch.bfloat16, torch.float16):
        x = torch.stack(rows).to(dt)
        w = torch.linspace(-1.0, 1.0, H).to(dt)
        w[::7] = -1.0
        rep, gpu = _run_and_compare(x, None, w, 1e-5, True)
        assert np.all(gpu["bs"].reshape(len(rows), H // 32)[0] == 0)    # zero row -> code 0
        _run_and_compare(x, torch.flip(x, [0]).contiguous(), w, 1e-5, True)


@pytest.mark.parametrize("M,H", [(1, 32), (33, 96), (129, 256), (300, 4096), (64, 5120),
                                 (5, 24576), (2, 32800), (2100, 512)])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_standalone_mxfp8_matches_oracle_exactly(M, H, dt):
    """The standalone quant is a function of y: codes and scales equal the
    oracle's bit for bit, on the vector path and (H > 32768 or an unaligned
    y) the scalar path; nothing is written past either output."""
    print(f"mxfp8 quant M={M} H={H} {dt}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M + H)
    spread = 4.0 if dt == torch.bfloat16 else 1.5     # fp16 kept inside its range
    y = (torch.randn(M, H, generator=g) * torch.exp(torch.randn(M, H // 32, 1, generator=g) * spread)
         .expand(M, H // 32, 32).reshape(M, H)).to(dt)
    assert bool(torch.isfinite(y).all())
    fmt = P.FMT[dt]
    qr, sr = O.quant_mxfp8(P.bits16(y), fmt)
    for off in (0, 2):
        ybuf = torch.zeros(M * H * 2 + off, dtype=torch.uint8, device=dev)
        yd = ybuf[off:].view(dt).view(M, H)
        yd.copy_(y.to(dev))
        qbuf = torch.full((M * H + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device=dev)
        sbuf = torch.full((M * (H // 32) + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device=dev)
        q, s = ops.quant_mxfp8(yd, qbuf[:M * H].view(ops.FP8_DTYPE).view(M, H),
                               sbuf[:M * (H // 32)].view(ops.E8M0_DTYPE).view(M, H // 32))
        torch.cuda.synchronize()
        assert np.array_equal(q.view(torch.uint8).cpu().numpy(), qr), off
        assert np.array_equal(s.view(torch.uint8).cpu().numpy(), sr), off
        assert bool((qbuf[M * H:] == P.SENTINEL).all()) and bool((sbuf[M * (H // 32):] == P.SENTINEL).all())


@pytest.mark.parametrize("name", ["nvfp4_prefill_m8192_h4096_bf16_y", "fp8_nores_m4096_h5120_fp16",
                                  "fp8_decode_m8_h4096_bf16"])
def test_mxfp8_unfused_chain_equals_fused(name):
    """add + norm (no quant), then the standalone MXFP8 quant of its y, gives
    the fused kernel's y, codes and scales bit for bit."""
    wl = WORKLOADS[name]
    print(f"mxfp8 unfused {name}", flush=True)
    x, r, w = make_inputs(wl)
    dev = torch.device("cuda")
    xd, wd = x.to(dev), w.to(dev)
    r1 = r.to(dev) if r is not None else None
    r2 = r.to(dev) if r is not None else None
    q1, s1, y1 = ops.add_rms_norm_quant(xd, r1, wd, wl.eps, None, "mxfp8", "gemma", True)
    y2 = ops.gemma_add_rms_norm(xd, r2, wd, wl.eps)
    q2, s2 = ops.quant_mxfp8(y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8))
    assert torch.equal(s1.view(torch.uint8), s2.view(torch.uint8))
    if r is not None:
        assert torch.equal(r1, r2)


def test_mxfp8_named_op_returns():
    """gemma_add_rms_norm_mxfp8 returns (codes, scales, normed or None,
    residual) with the shapes and dtypes of the MXFP8 variant."""
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(3)
    x = torch.randn(40, 1024, generator=g).to(torch.bfloat16).to(dev)
    r = torch.randn(40, 1024, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(1024, generator=g) * 0.1).to(torch.bfloat16).to(dev)
    q, s, y, res = ops.gemma_add_rms_norm_mxfp8(x, r, w, 1e-6, return_normed=True)
    assert q.shape == (40, 1024) and q.dtype == torch.float8_e4m3fn
    assert s.shape == (40, 32) and s.dtype == torch.float8_e8m0fnu
    assert y.shape == x.shape and res is r
    q0, s0, y0, _ = ops.gemma_add_rms_norm_mxfp8(x, None, w, 1e-6)
    assert y0 is None and q0.shape == (40, 1024)


def test_mxfp8_empty_batch_writes_nothing():
    dev = torch.device("cuda")
    buf = torch.full((8192,), P.SENTINEL, dtype=torch.uint8, device=dev)
    w = torch.zeros(128, dtype=torch.bfloat16, device=dev)
    p = buf.data_ptr()
    st = _lib.nq_add_rms_norm_quant(p, p + 1024, w.data_ptr(), 1e-6, 0, 0, 128, 0, 0,
                                    _lib.NQ_MODE_MXFP8, 1, p + 2048, p + 4096, p + 5120, 0)
    st2 = _lib.nq_quant_mxfp8(p, 0, 128, 0, p + 2048, p + 4096, 0)
    torch.cuda.synchronize()
    assert st == _lib.NQ_OK and st2 == _lib.NQ_OK and bool((buf == P.SENTINEL).all())


def test_mxfp8_deterministic():
    wl = WORKLOADS["nvfp4_prefill_m8192_h4096_bf16_y"]
    x, r, w = make_inputs(wl)
    a = P.run_gpu(x, r.clone(), w, wl.eps, 1.0, False, True, mxfp8=True)
    b = P.run_gpu(x, r.clone(), w, wl.eps, 1.0, False, True, mxfp8=True)
    for k in ("residual", "y", "q", "bs"):
        assert np.array_equal(a[k], b[k]), k


def test_mxfp8_scale_code_probe():
    """Kind 7: the kernel's E8M0 code of an fp32 amax equals the oracle's
    block rule, for every exponent with tie-heavy mantissas, powers of two
    and their neighbours, zeros and subnormals."""
    v = np.abs(_tie_heavy_f32(exp_lo=-149, exp_hi=127, n_random=300_000))
    extra = np.array([0.0, 2.0 ** -149, 2.0 ** -127, 2.0 ** -126, 2.0 ** -119, 448.0, 512.0,
                      np.nextafter(np.float32(512), np.float32(0)), 3.4e38], dtype=np.float32)
    v = np.concatenate([v, extra]).astype(np.float32)
    got = probe(7, v.view(np.uint32))
    want = (O.mxfp8_block_exponent(v.astype(np.float64)) + 127).astype(np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:6]]


@pytest.mark.parametrize("code", [0, 1, 100, 119, 120, 127, 128, 134, 200, 246, 247])
def test_mxfp8_element_probe(code):
    """Kind 8: the kernel's element code of fp32 v in a block with E8M0 scale
    code c equals E4M3FN_RNE(clamp(v * 2^(127 - c), +-448)) by the oracle,
    over every E4M3 tie (after scaling) and its neighbours."""
    # exponents whose scaled value spans E4M3's range, from below half its
    # smallest subnormal (2^-10) to beyond 448
    v = _tie_heavy_f32(exp_lo=max(-149, code - 127 - 12), exp_hi=min(127, code - 127 + 11),
                       n_random=100_000)
    got = probe(8, v.view(np.uint32), float(code))
    with np.errstate(over="ignore"):
        t = np.ldexp(v.astype(np.float64), 127 - code)
    want = O.encode(np.clip(t, -448, 448), O.E4M3FN)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(want[i])) for i in bad[:6]]
