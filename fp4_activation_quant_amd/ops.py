"""PyTorch-facing wrapper of the fused op, mirroring ``gemma_add_rms_norm_quant``
on the ``fused_norm_quant`` page: same arguments, same checks, same output
allocation (PyTorch provides device memory and the stream; the HIP library
does all the work)."""

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.NQ_BF16, torch.float16: _lib.NQ_FP16}
FP8_DTYPE = torch.float8_e4m3fn


def round_up(a, b):
    return (a + b - 1) // b * b


def _check(status, what):
    if status != _lib.NQ_OK:
        raise _lib.NqError(status, what)


def gemma_add_rms_norm_quant(x, residual, weight, eps, scale, nvfp4, write_y=False):
    """Gemma RMSNorm of ``x (+ residual)`` quantized for the next linear.

    x: (M, H) bf16/fp16, contiguous, read only.  residual: same shape or None;
    updated in place to x + residual.  weight: (H,); the norm scales by
    (1 + weight).  scale: fp32 tensor with one element -- FP8: the static
    per-tensor input scale; NVFP4: the global scale.  Returns
    ``(q, block_scale, y)``: FP8 codes (M, H) float8_e4m3fn, or packed E2M1
    (M, H // 2) uint8; NVFP4 block scales (round_up(M, 128),
    round_up(H // 16, 4)) float8_e4m3fn in the 128x4-tiled layout with rows
    >= M left unwritten, or ``scale`` for FP8; and the normed activation in
    x's dtype when ``write_y`` (else None).
    """
    assert x.dim() == 2 and x.is_contiguous()
    assert x.dtype in (torch.bfloat16, torch.float16)
    assert x.is_cuda
    assert residual is None or (residual.shape == x.shape and residual.is_contiguous()
                                and residual.dtype == x.dtype and residual.device == x.device)
    assert weight.shape == (x.shape[1],) and weight.is_contiguous() and weight.dtype == x.dtype
    assert scale.numel() == 1 and scale.dtype == torch.float32 and scale.device == x.device
    M, H = x.shape
    if nvfp4:
        assert H % 64 == 0
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=x.device)
        block_scale = torch.empty((round_up(M, 128), round_up(H // 16, 4) // 4),
                                  dtype=torch.int32, device=x.device).view(FP8_DTYPE)
    else:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=x.device)
        block_scale = scale
    y = torch.empty_like(x) if write_y else None
    if M == 0:
        return q, block_scale, y
    gemma_add_rms_norm_quant_out(x, residual, weight, eps, scale, nvfp4, q,
                                 block_scale if nvfp4 else None, y)
    return q, block_scale, y


def gemma_add_rms_norm_quant_out(x, residual, weight, eps, scale, nvfp4, q, block_scale, y):
    """Same op into caller-allocated outputs (no allocation, no checks beyond
    the library's own).  ``y`` None means write_y=False."""
    M, H = x.shape
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = _lib.nq_gemma_add_rms_norm_quant(
            x.data_ptr(), residual.data_ptr() if residual is not None else 0, weight.data_ptr(),
            eps, scale.data_ptr(), M, H, _DT[x.dtype],
            _lib.NQ_MODE_NVFP4 if nvfp4 else _lib.NQ_MODE_FP8_STATIC, y is not None,
            q.data_ptr(), block_scale.data_ptr() if block_scale is not None else 0,
            y.data_ptr() if y is not None else 0, stream)
    _check(st, "nq_gemma_add_rms_norm_quant")


def block_scale_bytes(M, H):
    return _lib.nq_block_scale_bytes(M, H)
