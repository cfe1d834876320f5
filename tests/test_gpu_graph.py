"""The op captured in a HIP graph (as bench.py --graph does): every replay,
with eager work and synchronisations between replays, must reproduce the
eager result bit for bit."""

import pytest
import torch

from fp4_activation_quant_amd import _lib, ops
from fp4_activation_quant_amd.workloads import WORKLOADS, make_inputs, load_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


@pytest.mark.parametrize("name", ["fp8_decode_m64_h4096_bf16", "nvfp4_res_m4096_h5120_fp16",
                                  "fp8_m16_h2048_bf16_y"])
def test_graph_replays_match_eager(name):
    print(f"graph {name}", flush=True)
    wl = WORKLOADS[name]
    dev = torch.device("cuda")
    x, r, w = make_inputs(wl)
    xd, wd = x.to(dev), w.to(dev)
    r0 = r.to(dev) if r is not None else None
    sd = torch.tensor([load_scale(wl)], dtype=torch.float32, device=dev)
    M, H = wl.M, wl.H

    def outputs():
        q = torch.full((M, H // 2 if wl.nvfp4 else H), 0x5A, dtype=torch.uint8, device=dev)
        bs = torch.full((ops.block_scale_bytes(M, H),), 0x5A, dtype=torch.uint8, device=dev) if wl.nvfp4 else None
        y = torch.zeros((M, H), dtype=x.dtype, device=dev)
        return q, bs, y

    # eager reference
    re = r0.clone() if r0 is not None else None
    qe, bse, ye = outputs()
    ops.gemma_add_rms_norm_quant_out(xd, re, wd, wl.eps, sd, wl.nvfp4,
                                     qe if wl.nvfp4 else qe.view(torch.float8_e4m3fn), bse, ye)
    torch.cuda.synchronize()

    rg = r0.clone() if r0 is not None else None
    qg, bsg, yg = outputs()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        ops.gemma_add_rms_norm_quant_out(xd, rg, wd, wl.eps, sd, wl.nvfp4,
                                         qg if wl.nvfp4 else qg.view(torch.float8_e4m3fn), bsg, yg)
    for rep in range(3):
        # eager work between replays: reset the in-place residual and outputs
        if rg is not None:
            rg.copy_(r0)
        qg.fill_(0x5A)
        if bsg is not None:
            bsg.fill_(0x5A)
        yg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qg, qe), rep
        assert torch.equal(yg, ye), rep
        if rg is not None:
            assert torch.equal(rg, re), rep
        if bsg is not None:
            assert torch.equal(bsg, bse), rep


@pytest.mark.parametrize("fmt,M,H,N", [("nvfp4", 4, 1024, 320), ("nvfp4", 40, 1152, 200),
                                       ("nvfp4", 300, 1024, 384), ("nvfp4", 300, 1024, 4096),
                                       ("nvfp4", 2100, 256, 4096), ("mxfp8", 300, 1024, 384),
                                       ("mxfp8", 2100, 512, 4096), ("mxfp8", 8, 2048, 4096),
                                       ("fp8", 8, 2048, 4096), ("fp8", 40, 1088, 200),
                                       ("fp8", 300, 1056, 384), ("fp8", 300, 1024, 384),
                                       ("fp8", 2100, 512, 4096)])
def test_graph_op_and_consumer_gemm_replays_match_eager(fmt, M, H, N):
    """The op and its consumer GEMM captured together (the NVFP4 dot-product,
    32 x 32, 128 x 64 and 256 x 256 tile kernels; the MXFP8 and static-FP8
    decode, 128 x 128 and 256 x 256 LDS-DMA kernels; the static-FP8 skinny
    and register-staged kernels): every replay, with eager resets and
    synchronisations between, gives the eager result bit for bit."""
    print(f"graph chain {fmt} M={M} H={H} N={N}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M + H + N)
    x = torch.randn(M, H, generator=g).to(torch.bfloat16).to(dev)
    r0 = torch.randn(M, H, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(H, generator=g) * 0.1).to(torch.bfloat16).to(dev)
    W = torch.randn(N, H, generator=g).to(torch.bfloat16).to(dev)
    gs = torch.tensor([448.0 * 6.0 / 9.0], dtype=torch.float32, device=dev)
    # static FP8: about 5 / 448 for the activation and the weight alike
    sa = torch.tensor([0.0125], dtype=torch.float32, device=dev)
    sb = torch.tensor([0.011], dtype=torch.float32, device=dev)
    if fmt == "nvfp4":
        wq, wbs = ops.quant_nvfp4(W, gs)
    elif fmt == "mxfp8":
        wq, wbs = ops.quant_mxfp8(W)
    else:
        wq = ops.quant_fp8_static(W, sb)

    def chain(r):
        if fmt == "nvfp4":
            q, bs, _ = ops.gemma_add_rms_norm_quant(x, r, w, 1e-6, gs, True)
            return ops.gemm_nvfp4(q, bs, gs, wq, wbs, gs)
        if fmt == "mxfp8":
            q, s, _, _ = ops.gemma_add_rms_norm_mxfp8(x, r, w, 1e-6)
            return ops.gemm_mxfp8(q, s, wq, wbs)
        q, _, _ = ops.gemma_add_rms_norm_quant(x, r, w, 1e-6, sa, False)
        return ops.gemm_fp8_static(q, sa, wq, sb)

    re = r0.clone()
    oute = chain(re)
    torch.cuda.synchronize()

    rg = r0.clone()
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=st):
        outg = chain(rg)
    for rep in range(3):
        rg.copy_(r0)
        outg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outg, oute), rep
        assert torch.equal(rg, re), rep


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,H", [(130, 2080), (7, 4096)])
def test_graph_unfused_chain_replays_match_eager(M, H, dtype):
    """The unfused chain (add + Gemma norm with no quant, then each standalone
    quant kernel) captured together: every replay, with eager resets and
    synchronisations between, writes the eager result bit for bit, NVFP4's
    untouched scale padding included."""
    print(f"graph unfused M={M} H={H} {dtype}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M * 3 + H)
    x = torch.randn(M, H, generator=g).to(dtype).to(dev)
    r0 = torch.randn(M, H, generator=g).to(dtype).to(dev)
    w = (torch.randn(H, generator=g) * 0.1).to(dtype).to(dev)
    s8 = torch.tensor([0.0125], dtype=torch.float32, device=dev)
    gs = torch.tensor([448.0 * 6.0 / 9.0], dtype=torch.float32, device=dev)

    def outputs():
        return {"q8": torch.empty((M, H), dtype=torch.uint8, device=dev),
                "q4": torch.empty((M, H // 2), dtype=torch.uint8, device=dev),
                "bs4": torch.empty((_lib.nq_block_scale_bytes(M, H),), dtype=torch.uint8, device=dev),
                "qmx": torch.empty((M, H), dtype=torch.uint8, device=dev),
                "smx": torch.empty((M, H // 32), dtype=torch.uint8, device=dev)}

    def chain(r, o):
        _, _, y = ops.add_rms_norm_quant(x, r, w, 1e-6, None, None)
        ops.quant_fp8_static(y, s8, o["q8"].view(torch.float8_e4m3fn))
        ops.quant_nvfp4(y, gs, o["q4"], o["bs4"].view(torch.float8_e4m3fn))
        ops.quant_mxfp8(y, o["qmx"].view(torch.float8_e4m3fn), o["smx"].view(torch.float8_e8m0fnu))
        return y

    def reset(r, o):
        r.copy_(r0)
        for t in o.values():
            t.fill_(0xA5)

    re, oe = r0.clone(), outputs()
    reset(re, oe)
    ye = chain(re, oe)
    torch.cuda.synchronize()

    rg, og = r0.clone(), outputs()
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=st):
        yg = chain(rg, og)
    for rep in range(3):
        reset(rg, og)
        yg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), rep
        assert torch.equal(rg, re), rep
        for k in oe:
            assert torch.equal(og[k], oe[k]), (rep, k)


@pytest.mark.parametrize("M", [2, 6])
def test_graph_decode_step_replays_match_eager(M):
    """The decode step (one launch at M = 2, the op and the decode GEMM at
    M = 6) captured in a graph: every replay, with eager work between them,
    reproduces the eager outputs bit for bit."""
    print(f"graph decode step M={M}", flush=True)
    import numpy as np
    dev = torch.device("cuda")
    H = N = 4096
    g0 = torch.Generator().manual_seed(4200 + M)
    x = torch.randn(M, H, generator=g0).to(torch.bfloat16).to(dev)
    r = (torch.randn(M, H, generator=g0) * 2).to(torch.bfloat16).to(dev)
    w = (torch.randn(H, generator=g0) * 0.1).to(torch.bfloat16).to(dev)
    s = torch.tensor([0.02], dtype=torch.float32, device=dev)
    bs = torch.tensor([0.004], dtype=torch.float32, device=dev)
    rng = np.random.default_rng(M)
    b = torch.from_numpy((rng.integers(0, 8, size=(N, H)) | (rng.integers(0, 8, size=(N, H)) << 3)
                          | (rng.integers(0, 2, size=(N, H)) << 7)).astype(np.uint8)).to(dev)

    def outputs():
        return (torch.full((M, H), 0x5A5A, dtype=torch.int16, device=dev).view(torch.bfloat16),
                torch.full((M, H), 0x5A, dtype=torch.uint8, device=dev),
                torch.zeros((M, H), dtype=torch.bfloat16, device=dev),
                torch.zeros((M, N), dtype=torch.bfloat16, device=dev))

    ro, q, y, out = outputs()
    ops.gemma_add_rms_norm_quant_gemm_fp8_out(x, r, ro, w, 1e-6, s, b, bs, q, y, out)
    torch.cuda.synchronize()
    want = [t.clone() for t in (ro, q, y, out)]

    rog, qg, yg, outg = outputs()
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=st):
        ops.gemma_add_rms_norm_quant_gemm_fp8_out(x, r, rog, w, 1e-6, s, b, bs, qg, yg, outg)
    for rep in range(3):
        for t in (rog, yg, outg):
            t.zero_()
        qg.fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((rog, qg, yg, outg), want):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), rep
