"""The GPU-vs-oracle comparison itself, on the CPU: fed a "GPU" result that
the oracle wrote, it reports no difference; with one planted wrong byte in
a code, a y value or a block scale, it reports exactly that difference.
The chunked, threaded aggregation is checked against a single-chunk run."""

import numpy as np
import pytest
import torch

import oracle as O
from tests import parity as P


def _fake_gpu(x, r, w, eps, scale, mode, write_y=True):
    fmt = P.FMT[x.dtype]
    M, H = x.shape
    ref = O.add_rms_norm_quant(P.bits16(x), P.bits16(r) if r is not None else None, P.bits16(w), eps,
                               scale, mode, "gemma", fmt)
    bs = None
    if mode == "nvfp4":
        bs = ref["block_scale"].copy()
    elif mode == "mxfp8":
        bs = ref["scales"].reshape(-1).copy()
    return {"M": M, "H": H, "nvfp4": mode == "nvfp4", "dtype": x.dtype, "mode": mode, "norm": "gemma",
            "x_unchanged": True, "residual": ref["residual"], "y": ref["y"].copy() if write_y else None,
            "q": ref["q"].copy(), "bs": bs, "guards_ok": True}


def _inputs(M, H, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    r = torch.randn(M, H, generator=g).to(torch.bfloat16)
    w = (torch.randn(H, generator=g) * 0.1).to(torch.bfloat16)
    return x, r, w


@pytest.mark.parametrize("mode,scale", [("fp8", 0.02), ("nvfp4", 448 * 6 / 5.0), ("mxfp8", 1.0)])
def test_clean_run_passes_and_chunking_agrees(mode, scale):
    x, r, w = _inputs(300, 256, 3)
    gpu = _fake_gpu(x, r, w, 1e-6, scale, mode)
    rep = P.check(P.compare(gpu, x, r, w, 1e-6, scale, P.all_rows(300), threads=4))
    assert rep["rows"] == 300 and rep["code_diff_fraction"] == 0 and rep.get("y_max_ulp", 0) == 0
    if mode != "fp8":
        assert rep["scale_match_fraction"] == 1.0
    one = P.compare(gpu, x, r, w, 1e-6, scale, P.all_rows(300), threads=1)
    assert one == rep
    if mode == "nvfp4":
        assert rep["padding_written"] == 0      # rows 300..383 of the scale buffer


def test_planted_code_y_and_scale_differences_are_found():
    x, r, w = _inputs(260, 128, 5)
    gs = 448 * 6 / 5.0
    gpu = _fake_gpu(x, r, w, 1e-6, gs, "nvfp4")
    # one code nibble one step off in the last row (a chunk of its own)
    q = gpu["q"]
    lo = q[259, 3] & 0xF
    q[259, 3] = (q[259, 3] & 0xF0) | (lo + 1 if (lo & 7) < 7 else lo - 1)
    rep = P.compare(gpu, x, r, w, 1e-6, gs, P.all_rows(260), threads=3)
    assert rep["code_max_step"] == 1 and rep["code_diff_fraction"] == pytest.approx(1 / (260 * 128))
    assert rep["code_mismatch_where_y_equal"] == 1 and rep["requant_code_mismatch"] == 1
    with pytest.raises(AssertionError):
        P.check(rep)
    # one y value two units off in row 128 (the second chunk)
    gpu = _fake_gpu(x, r, w, 1e-6, gs, "nvfp4")
    gpu["y"][128, 7] = np.uint16(int(gpu["y"][128, 7]) + 2)
    rep = P.compare(gpu, x, r, w, 1e-6, gs, P.all_rows(260), threads=3)
    assert rep["y_max_ulp"] == 2
    # one block scale changed in row 200 and a padding byte written
    gpu = _fake_gpu(x, r, w, 1e-6, gs, "nvfp4")
    off = int(O.swizzle_128x4_offset(200, 5, 128))
    gpu["bs"][off] ^= 1
    off_pad = int(O.swizzle_128x4_offset(300, 0, 128))
    gpu["bs"][off_pad] = 0
    rep = P.compare(gpu, x, r, w, 1e-6, gs, P.all_rows(260), threads=3)
    assert rep["scale_match_fraction"] == pytest.approx(1 - 1 / (260 * 8))
    assert rep["scale_mismatch_where_y_equal"] == 1 and rep["padding_written"] == 1


def test_missing_residual_row_is_found():
    x, r, w = _inputs(140, 64, 9)
    gpu = _fake_gpu(x, r, w, 1e-6, 0.05, "fp8", write_y=False)
    gpu["residual"] = gpu["residual"].copy()
    gpu["residual"][139] = 0xA5A5
    rep = P.compare(gpu, x, r, w, 1e-6, 0.05, P.all_rows(140), threads=2)
    assert rep["residual_mismatch"] == 64
    assert "y_max_ulp" not in rep
