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
