"""GPU parity: the HIP op against the CPU oracle, through the C ABI.

Every workload runs at its full size in the launch configuration the
benchmark uses; the oracle checks every row of every output (threaded over
128-row chunks), plus residual == x + residual by torch's CPU add, guard
bytes and untouched scale padding.  Edge cases cover
ragged tiles, the scalar path (H % 16 != 0, H > 32768, unaligned views),
1, 2 and 4 chunks per thread, the looping launch with early loads (4096 < H
< 6144 at 2048 <= M <= 16384), several rows per wave (H <= 512),
residual=None, write_y off, special values, M == 0,
determinism and argument errors.
"""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib, ops
from fp4_activation_quant_amd.workloads import WORKLOADS, make_inputs, load_scale
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()  # the HIP library must be there: no fallback


def _run_and_compare(x, r, w, eps, scale, nvfp4, write_y, rows=None, misalign=False, mxfp8=False):
    r_in = r.clone() if r is not None else None
    gpu = P.run_gpu(x, r_in, w, eps, scale, nvfp4, write_y, misalign=misalign, mxfp8=mxfp8)
    y_gpu = None
    if not write_y:
        # The same kernel arithmetic with y written, for the quant-step check.
        y_gpu = P.run_gpu(x, r.clone() if r is not None else None, w, eps, scale, nvfp4, True,
                          misalign=misalign, mxfp8=mxfp8)["y"]
    M = x.shape[0]
    rows = P.all_rows(M) if rows is None else rows
    rep = P.compare(gpu, x, r, w, eps, scale, rows, y_gpu=y_gpu)
    if r is not None:
        rep["residual_full_mismatch"] = int(np.count_nonzero(gpu["residual"] != P.bits16(x + r)))
        assert rep["residual_full_mismatch"] == 0
    print(rep, flush=True)
    return P.check(rep), gpu


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    wl = WORKLOADS[name]
    print(f"workload {name}", flush=True)
    x, r, w = make_inputs(wl)
    rep, _ = _run_and_compare(x, r, w, wl.eps, load_scale(wl), wl.nvfp4, wl.write_y, rows=P.all_rows(wl.M),
                              mxfp8=wl.mode == "mxfp8")
    P.record(name, rep)


EDGE = [
    # dtype, nvfp4, M, H, residual, write_y
    (torch.bfloat16, False, 1, 64, True, True),
    (torch.bfloat16, False, 127, 2048, True, True),
    (torch.bfloat16, False, 129, 5120, False, False),
    (torch.bfloat16, False, 300, 80, True, True),        # H % 16 != 0: scalar path
    (torch.bfloat16, False, 65, 1000, True, False),      # scalar path
    (torch.bfloat16, False, 3, 16384, True, True),       # 2 chunks x 1024 threads
    (torch.bfloat16, False, 5, 20480, True, True),       # 4 chunks per thread
    (torch.bfloat16, False, 9, 4112, True, True),        # one chunk per thread, a partial last wave
    (torch.bfloat16, False, 9, 4112, False, True),       # ragged: some threads own 1 chunk
    (torch.bfloat16, False, 33, 48, True, True),         # 6 chunks, one partial wave
    (torch.bfloat16, False, 2, 40000, True, True),       # H > 32768: scalar path
    (torch.float16, False, 257, 4096, True, True),
    (torch.bfloat16, True, 1, 64, True, True),
    (torch.bfloat16, True, 127, 128, True, True),
    (torch.bfloat16, True, 129, 2048, True, False),
    (torch.bfloat16, True, 257, 4096, False, True),
    (torch.bfloat16, True, 130, 16384, True, True),
    (torch.bfloat16, True, 3, 32768, True, True),        # 4 chunks x 1024 threads
    (torch.float16, True, 3, 32832, True, True),         # NVFP4 beyond 32768: scalar path
    (torch.bfloat16, True, 17, 4160, True, True),        # one chunk per thread (residual, H <= 5120)
    (torch.bfloat16, True, 17, 4160, False, True),       # ragged 2-chunk split
    (torch.bfloat16, True, 2100, 256, True, True),       # XCD row map: 2 spans + ragged tail
    (torch.float16, True, 3072, 64, False, True),        # XCD row map: exact spans
    (torch.float16, True, 200, 5120, True, True),
    (torch.float16, True, 2100, 5120, True, True),       # row loop with prefetch, ragged
    (torch.bfloat16, False, 3000, 4160, False, False),   # row loop with prefetch
    (torch.bfloat16, True, 45, 6144, True, True),        # one chunk per thread, 12 waves
    (torch.float16, False, 33, 8192, False, True),       # one chunk per thread, 16 waves
    (torch.float16, True, 64, 192, False, False),
    # H <= 512: several rows per wave (lanes per row 2, 4, 8, 16, 32, 64)
    (torch.bfloat16, False, 37, 16, True, True),
    (torch.bfloat16, False, 300, 32, True, False),
    (torch.float16, False, 1, 112, True, True),
    (torch.bfloat16, False, 129, 256, False, True),
    (torch.bfloat16, False, 65, 496, True, True),
    (torch.float16, False, 1000, 512, True, False),
    (torch.bfloat16, True, 37, 128, True, True),
    (torch.float16, True, 1, 320, True, True),
    (torch.bfloat16, True, 1000, 448, False, True),
    (torch.bfloat16, True, 255, 512, True, False),
]


@pytest.mark.parametrize("dt,nvfp4,M,H,res,wy", EDGE)
def test_edge_shapes(dt, nvfp4, M, H, res, wy):
    print(f"edge {dt} nvfp4={nvfp4} M={M} H={H} res={res} write_y={wy}", flush=True)
    g = torch.Generator().manual_seed(M * 7919 + H)
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt) if res else None
    w = (torch.randn(H, generator=g) * 0.2).to(dt)
    scale = 0.03 if not nvfp4 else 448 * 6 / 5.0
    _run_and_compare(x, r, w, 1e-6, scale, nvfp4, wy)


PREFETCH = [
    # dtype, output, M, H, residual, write_y: rows of 4096 < H < 6144 at
    # 2048 <= M <= 16384 loop 1024 (or 512) workgroups over the rows
    (torch.float16, "nvfp4", 2100, 5120, True, True),
    (torch.bfloat16, "nvfp4", 2049, 4864, True, True),    # one row past the last full 1024-row span
    (torch.float16, "mxfp8", 2050, 4224, False, True),    # some threads own one chunk
    (torch.bfloat16, "fp8", 4096, 5120, True, True),
    (torch.bfloat16, "mxfp8", 2100, 5120, False, True),  # no residual, threads covering the row: no guards
    (torch.float16, "nvfp4", 16384, 5120, False, False),
    (torch.bfloat16, "fp8", 3000, 4160, False, False),
    (torch.float16, "nvfp4", 4096, 6080, False, False),
    (torch.bfloat16, "nvfp4", 16384, 5120, True, False),
    (torch.bfloat16, "mxfp8", 2100, 5120, True, False),
    (torch.float16, "none", 2048, 4608, True, True),      # add + plain norm alone
    (torch.bfloat16, "fp8", 2048, 5120, False, True),     # no guards; static FP8 by the fp32 division
    (torch.float16, "fp8", 2049, 5120, False, False),     # no guards; static FP8 on packed fp16 halves
    (torch.bfloat16, "nvfp4", 2048, 5120, True, False),   # 512 workgroups, 4 rows each
    (torch.float16, "nvfp4", 8192, 4352, True, True),     # 512 workgroups, 16 rows each
    (torch.float16, "nvfp4", 6144, 5120, False, True),    # 1024 workgroups, 6 rows each
]


@pytest.mark.parametrize("dt,out,M,H,res,wy", PREFETCH)
def test_row_loop_matches_one_workgroup_per_row(dt, out, M, H, res, wy):
    """Rows are independent, so every byte the looping launch writes (the
    whole residual, y, codes and scale buffer) must equal that of 1024-row
    slices, which launch one workgroup per row; both launch forms are
    checked against the oracle, every row, by the other tests."""
    print(f"prefetch loop {dt} {out} M={M} H={H} res={res} write_y={wy}", flush=True)
    g = torch.Generator().manual_seed(M * 31 + H)
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt) if res else None
    w = (torch.randn(H, generator=g) * 0.2).to(dt)
    nvfp4 = out == "nvfp4"
    scale = 0.03 if not nvfp4 else 448 * 6 / 5.0
    kw = dict(mxfp8=out == "mxfp8", quant=out != "none", norm="plain" if out == "none" else "gemma")

    def run(a, b):
        return P.run_gpu(x[a:b], r[a:b].clone() if res else None, w, 1e-6, scale, nvfp4, wy, **kw)

    full = run(0, M)
    assert full["guards_ok"]
    tile_row = ops.block_scale_bytes(128, H)      # bytes of one 128-row band of scale tiles
    for a in range(0, M, 1024):
        b = min(M, a + 1024)
        part = run(a, b)
        for k in ("residual", "y", "q"):
            if full[k] is not None:
                assert np.array_equal(full[k][a:b], part[k]), (k, a)
        if nvfp4:
            o = a // 128 * tile_row
            assert np.array_equal(full["bs"][o:o + part["bs"].size], part["bs"]), a
        elif out == "mxfp8":
            assert np.array_equal(full["bs"].reshape(M, H // 32)[a:b].ravel(), part["bs"]), a


@pytest.mark.parametrize("nvfp4", [False, True])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_unaligned_views_take_the_scalar_path(nvfp4, dt):
    print(f"unaligned nvfp4={nvfp4} {dt}", flush=True)
    g = torch.Generator().manual_seed(99)
    M, H = 70, 256
    x = torch.randn(M, H, generator=g).to(dt)
    r = torch.randn(M, H, generator=g).to(dt)
    w = (torch.randn(H, generator=g) * 0.2).to(dt)
    _run_and_compare(x, r, w, 1e-6, 0.02 if not nvfp4 else 300.0, nvfp4, True, misalign=True)


def _special_rows(H, dt):
    rows = [
        torch.zeros(H),                                   # zero row (eps > 0 -> y = 0)
        torch.full((H,), 3.0),                            # constant row
        torch.full((H,), -2.0 ** -10),                    # small constant
        torch.linspace(-1000, 1000, H),                   # wide range
        torch.where(torch.arange(H) % 2 == 0, 1e4, -1e-3),
    ]
    return torch.stack(rows).to(dt)


@pytest.mark.parametrize("nvfp4", [False, True])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_special_values(nvfp4, dt):
    print(f"special nvfp4={nvfp4} {dt}", flush=True)
    H = 256
    x = _special_rows(H, dt)
    w = torch.linspace(-1.0, 1.0, H).to(dt)
    w[::7] = -1.0                                          # 1 + w == 0 columns
    # FP8: a tiny scale saturates most codes; NVFP4: a large global scale
    # saturates the block scales.
    for scale in ((1e-3, 0.5) if not nvfp4 else (1e5, 2.0)):
        _run_and_compare(x, None, w, 1e-5, scale, nvfp4, True)
        _run_and_compare(x, torch.flip(x, [0]).contiguous(), w, 1e-5, scale, nvfp4, True)


ZERO_SIGN_SHAPES = [
    # M, H, misaligned views: every launch form
    (9, 256, False),       # several rows per wave
    (9, 1024, False),      # one workgroup per row
    (2048, 5120, False),   # the looping launch
    (9, 1000, False),      # element-wise path (H % 16 != 0)
    (9, 1024, True),       # element-wise path (unaligned views)
]


@pytest.mark.parametrize("M,H,misalign", ZERO_SIGN_SHAPES)
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("norm", ["gemma", "plain"])
def test_zero_products_keep_their_sign(M, H, misalign, dt, norm):
    """y = t * g is an exact zero where the norm factor g is (w = -1 for
    Gemma's 1 + w, w = 0 for the plain norm) or where h is (x = -residual
    gives h = +0): IEEE gives it the product's sign, and the codes keep it
    (0x80 / 0x8 for -0).  The fp16 element-wise kernel once rounded such a
    product with a fused multiply-add of +0, which returns +0 for a -0
    product."""
    print(f"zero products M={M} H={H} misalign={misalign} {dt} {norm}", flush=True)
    g = torch.Generator().manual_seed(M * 17 + H + (1 if norm == "plain" else 0))
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt)
    r[0] = -x[0]                                        # h = +0 across row 0
    w = (torch.randn(H, generator=g) * 0.3).to(dt)
    w[::5] = -1.0 if norm == "gemma" else 0.0           # zero norm factor
    for mode in ("fp8", "nvfp4", "mxfp8", "none"):
        if (mode == "nvfp4" and H % 64) or (mode == "mxfp8" and H % 32):
            continue
        scale = {"fp8": 0.02, "nvfp4": 448 * 6 / 8.0}.get(mode, 1.0)
        for res in (r, None):
            gpu = P.run_gpu(x, res.clone() if res is not None else None, w, 1e-6, scale, mode == "nvfp4", True,
                            misalign=misalign, norm=norm, quant=mode != "none", mxfp8=mode == "mxfp8")
            P.check(P.compare(gpu, x, res, w, 1e-6, scale, P.all_rows(M)))


def test_empty_batch_launches_nothing():
    dev = torch.device("cuda")
    for nvfp4 in (False, True):
        x = torch.empty(0, 128, dtype=torch.bfloat16, device=dev)
        w = torch.zeros(128, dtype=torch.bfloat16, device=dev)
        s = torch.ones(1, dtype=torch.float32, device=dev)
        q, bs, y = ops.gemma_add_rms_norm_quant(x, x.clone(), w, 1e-6, s, nvfp4, True)
        assert q.shape[0] == 0 and y.shape == (0, 128)
        # raw call with M = 0 on live buffers writes nothing
        buf = torch.full((4096,), P.SENTINEL, dtype=torch.uint8, device=dev)
        st = _lib.nq_gemma_add_rms_norm_quant(
            buf.data_ptr(), buf.data_ptr() + 1024, w.data_ptr(), 1e-6, s.data_ptr(), 0, 128, 0,
            int(nvfp4), 1, buf.data_ptr() + 2048, buf.data_ptr() + 3072, buf.data_ptr() + 3584, 0)
        torch.cuda.synchronize()
        assert st == _lib.NQ_OK and bool((buf == P.SENTINEL).all())


def test_deterministic_across_runs():
    wl = WORKLOADS["nvfp4_prefill_m8192_h4096_bf16_y"]
    x, r, w = make_inputs(wl)
    a = P.run_gpu(x, r.clone(), w, wl.eps, load_scale(wl), True, True)
    b = P.run_gpu(x, r.clone(), w, wl.eps, load_scale(wl), True, True)
    for k in ("residual", "y", "q", "bs"):
        assert np.array_equal(a[k], b[k]), k
    wl = WORKLOADS["fp8_res_m4096_h5120_fp16"]
    x, r, w = make_inputs(wl)
    a = P.run_gpu(x, r.clone(), w, wl.eps, load_scale(wl), False, True)
    b = P.run_gpu(x, r.clone(), w, wl.eps, load_scale(wl), False, True)
    for k in ("residual", "y", "q"):
        assert np.array_equal(a[k], b[k]), k


def test_invalid_arguments_write_nothing():
    dev = torch.device("cuda")
    M, H = 4, 128
    buf = torch.full((1 << 16,), P.SENTINEL, dtype=torch.uint8, device=dev)
    s = torch.ones(1, dtype=torch.float32, device=dev)
    p = buf.data_ptr()
    x, r, w, q, bs, y = p, p + 4096, p + 8192, p + 12288, p + 16384, p + 24576
    call = _lib.nq_gemma_add_rms_norm_quant
    cases = [
        (dict(x=0), _lib.NQ_EINVAL),
        (dict(w=0), _lib.NQ_EINVAL),
        (dict(s=0), _lib.NQ_EINVAL),
        (dict(q=0), _lib.NQ_EINVAL),
        (dict(M=-1), _lib.NQ_EINVAL),
        (dict(H=0), _lib.NQ_EINVAL),
        (dict(dtype=2), _lib.NQ_EINVAL),
        (dict(mode=2), _lib.NQ_EINVAL),
        (dict(wy=1, y=0), _lib.NQ_EINVAL),
        (dict(mode=1, bs=0), _lib.NQ_EINVAL),
        (dict(mode=1, H=80), _lib.NQ_EUNSUPPORTED),
        (dict(r=p), _lib.NQ_EINVAL),                 # residual aliases x
        (dict(q=p + 4096 + 512), _lib.NQ_EINVAL),    # q overlaps residual
        (dict(q=p + 8192 + 64), _lib.NQ_EINVAL),     # q overlaps the weight
        (dict(r=p + 8192 - 1022), _lib.NQ_EINVAL),   # residual reaches into the weight
        (dict(wy=1, y=p + 8192 + 200), _lib.NQ_EINVAL),
        (dict(mode=1, bs=p + 8192), _lib.NQ_EINVAL),
        (dict(s=p + 12288 + 8), _lib.NQ_EINVAL),     # the scale inside q
        (dict(mode=1, s=p + 16384 + 4), _lib.NQ_EINVAL),  # the global scale inside the scales
    ]
    for over, want in cases:
        a = dict(x=x, r=r, w=w, s=s.data_ptr(), M=M, H=H, dtype=0, mode=0, wy=0, q=q, bs=bs, y=y)
        a.update(over)
        st = call(a["x"], a["r"], a["w"], 1e-6, a["s"], a["M"], a["H"], a["dtype"], a["mode"],
                  a["wy"], a["q"], a["bs"], a["y"], 0)
        assert st == want, (over, st)
    torch.cuda.synchronize()
    assert bool((buf == P.SENTINEL).all())


def test_read_only_inputs_may_share_memory():
    """x, the weight and the scale are only read, so they may overlap: the
    weight here is x's first row and the fp32 scale is two bf16 elements of
    x's row 5."""
    M, H = 64, 1024
    g = torch.Generator().manual_seed(77)
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    r = torch.randn(M, H, generator=g).to(torch.bfloat16)
    sv = torch.tensor([0.04], dtype=torch.float32)
    x[5, 10:12] = sv.view(torch.bfloat16)               # the scale's bytes inside x
    dev = torch.device("cuda")
    xd, rd = x.to(dev), r.to(dev)
    q = torch.empty((M, H), dtype=torch.uint8, device=dev)
    y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    st = _lib.nq_gemma_add_rms_norm_quant(xd.data_ptr(), rd.data_ptr(), xd.data_ptr(), 1e-6,
                                          xd.data_ptr() + (5 * H + 10) * 2, M, H, 0, 0, 1,
                                          q.data_ptr(), 0, y.data_ptr(), 0)
    assert st == _lib.NQ_OK
    torch.cuda.synchronize()
    ref = O.gemma_add_rms_norm_quant(P.bits16(x), P.bits16(r), P.bits16(x[0].clone()), 1e-6,
                                     float(sv[0]), False, True)
    assert np.array_equal(P.bits16(rd), ref["residual"])
    dy = np.abs(P._ord16(P.bits16(y)) - P._ord16(ref["y"]))
    assert dy.max() <= 1
    same = P.bits16(y) == ref["y"]
    assert np.array_equal(q.cpu().numpy()[same], ref["q"][same])


def test_runs_on_the_callers_stream():
    wl = WORKLOADS["fp8_m16_h2048_bf16_y"]
    x, r, w = make_inputs(wl)
    dev = torch.device("cuda")
    s = torch.tensor([load_scale(wl)], dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    xd, rd, wd = x.to(dev), r.to(dev), w.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        q, _, y = ops.gemma_add_rms_norm_quant(xd, rd, wd, wl.eps, s, False, True)
    side.synchronize()
    ref = O.gemma_add_rms_norm_quant(P.bits16(x), P.bits16(r), P.bits16(w), wl.eps, load_scale(wl),
                                     False, True, O.BF16)
    assert np.array_equal(P.bits16(rd), ref["residual"])
    assert np.max(np.abs(P._ord16(P.bits16(y)) - P._ord16(ref["y"]))) <= 1
