"""GPU parity of the op's variants and of its unfused form, through the C ABI:
plain RMSNorm (scale by w), add + norm without quant, the standalone FP8 /
NVFP4 quant kernels, and the unfused chain (add + norm, then quant) run on
the GPU, which must reproduce the fused kernel's outputs bit for bit."""

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
    _lib.lib()


def _inputs(M, H, dt, res, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g).to(dt)
    r = (torch.randn(M, H, generator=g) * 2).to(dt) if res else None
    w = (torch.randn(H, generator=g) * 0.3 + 1.0).to(dt)
    return x, r, w


SHAPES = [(1, 64), (37, 256), (129, 2048), (300, 5120), (5, 20480), (65, 1000)]


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("mode", ["fp8", "nvfp4", None])
@pytest.mark.parametrize("norm", ["plain", "gemma"])
def test_variant_parity(M, H, mode, norm):
    if mode == "nvfp4" and H % 64:
        pytest.skip("NVFP4 needs H % 64 == 0")
    if mode == "fp8" and norm == "gemma":
        pytest.skip("covered by test_gpu_parity")
    print(f"variant M={M} H={H} mode={mode} norm={norm}", flush=True)
    for dt, res in ((torch.bfloat16, True), (torch.float16, False)):
        x, r, w = _inputs(M, H, dt, res, M * 131 + H)
        scale = {"fp8": 0.02, "nvfp4": 448 * 6 / 8.0, None: 1.0}[mode]
        gpu = P.run_gpu(x, r.clone() if r is not None else None, w, 1e-6, scale, mode == "nvfp4",
                        True, norm=norm, quant=mode is not None)
        rep = P.check(P.compare(gpu, x, r, w, 1e-6, scale, P.all_rows(M)))
        print(rep, flush=True)


@pytest.mark.parametrize("M,H", [(1, 16), (33, 48), (129, 256), (300, 4096), (64, 5120), (7, 1000),
                                 (2100, 512)])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_standalone_quant_matches_oracle_exactly(M, H, dt):
    """The quant step alone is a function of y: codes and scales must equal
    the oracle's bit for bit (FP8 any H; NVFP4 H % 16 == 0, including a
    partial last 4-column scale tile)."""
    print(f"quant M={M} H={H} {dt}", flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(M + H)
    y = (torch.randn(M, H, generator=g) * torch.exp(torch.randn(M, 1, generator=g))).to(dt)
    yd = y.to(dev)
    fmt = P.FMT[dt]
    s = torch.tensor([0.0137], dtype=torch.float32, device=dev)
    q = ops.quant_fp8_static(yd, s)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(),
                          O.quant_fp8_static(P.bits16(y), fmt, float(s.item())))
    if H % 16 == 0:
        gs = torch.tensor([448 * 6 / 9.0], dtype=torch.float32, device=dev)
        nb = ops.block_scale_bytes(M, H)
        bs = torch.full((nb,), P.SENTINEL, dtype=torch.uint8, device=dev)
        qn, _ = ops.quant_nvfp4(yd, gs, block_scale=bs)
        qr, S = O.quant_nvfp4(P.bits16(y), fmt, float(gs.item()))
        assert np.array_equal(qn.cpu().numpy(), qr)
        want = np.full(nb, P.SENTINEL, np.uint8)
        O.scatter_block_scales(S, M, H, want)
        assert np.array_equal(bs.cpu().numpy(), want)   # padding rows/columns untouched


@pytest.mark.parametrize("name", ["nvfp4_prefill_m8192_h4096_bf16_y", "fp8_res_m4096_h5120_fp16",
                                  "nvfp4_nores_m4096_h5120_fp16", "fp8_decode_m64_h4096_bf16"])
def test_unfused_chain_equals_fused(name):
    """add + Gemma norm (no quant) followed by the standalone quant, on the
    GPU, gives the fused kernel's residual, y, codes and scales bit for bit
    (the page: the fused kernel's codes match the unfused chain)."""
    print(f"unfused {name}", flush=True)
    wl = WORKLOADS[name]
    dev = torch.device("cuda")
    x, r, w = make_inputs(wl)
    xd, wd = x.to(dev), w.to(dev)
    sd = torch.tensor([load_scale(wl)], dtype=torch.float32, device=dev)
    r1 = r.to(dev) if r is not None else None
    r2 = r.to(dev) if r is not None else None
    # fused
    q1, bs1, y1 = ops.gemma_add_rms_norm_quant(xd, r1, wd, wl.eps, sd, wl.nvfp4, True)
    # unfused: add + norm, then the standalone quant of y
    y2 = ops.gemma_add_rms_norm(xd, r2, wd, wl.eps)
    if wl.nvfp4:
        q2, bs2 = ops.quant_nvfp4(y2, sd)
    else:
        q2 = ops.quant_fp8_static(y2, sd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8))
    if r is not None:
        assert torch.equal(r1, r2) and torch.equal(r2.cpu(), x + r)
    if wl.nvfp4:
        mm, bb = np.meshgrid(np.arange(wl.M), np.arange(wl.H // 16), indexing="ij")
        idx = torch.from_numpy(O.swizzle_128x4_offset(mm, bb, wl.H).reshape(-1)).to(dev)
        b1, b2 = bs1.view(torch.uint8).flatten(), bs2.view(torch.uint8).flatten()
        assert torch.equal(b1[idx], b2[idx])
