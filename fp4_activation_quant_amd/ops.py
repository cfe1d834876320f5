"""PyTorch-facing wrapper of the fused op, mirroring ``gemma_add_rms_norm_quant``
on the ``fused_norm_quant`` page: same arguments, same checks, same output
allocation (PyTorch provides device memory and the stream; the HIP library
does all the work)."""

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.NQ_BF16, torch.float16: _lib.NQ_FP16}
FP8_DTYPE = torch.float8_e4m3fn
E8M0_DTYPE = torch.float8_e8m0fnu


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


def _ptr(t):
    return t.data_ptr() if t is not None else 0


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def gemma_add_rms_norm_quant_out(x, residual, weight, eps, scale, nvfp4, q, block_scale, y):
    """Same op into caller-allocated outputs (no allocation, no checks beyond
    the library's own).  ``y`` None means write_y=False."""
    M, H = x.shape
    with torch.cuda.device(x.device):
        st = _lib.nq_gemma_add_rms_norm_quant(
            x.data_ptr(), _ptr(residual), weight.data_ptr(), eps, scale.data_ptr(), M, H,
            _DT[x.dtype], _lib.NQ_MODE_NVFP4 if nvfp4 else _lib.NQ_MODE_FP8_STATIC, y is not None,
            q.data_ptr(), _ptr(block_scale), _ptr(y), _stream(x.device))
    _check(st, "nq_gemma_add_rms_norm_quant")


_MODES = {"fp8": _lib.NQ_MODE_FP8_STATIC, "nvfp4": _lib.NQ_MODE_NVFP4, "mxfp8": _lib.NQ_MODE_MXFP8,
          None: _lib.NQ_MODE_NONE}
_NORMS = {"gemma": _lib.NQ_NORM_GEMMA, "plain": _lib.NQ_NORM_PLAIN}


def add_rms_norm_quant_out(x, residual, weight, eps, scale, mode, norm, q, block_scale, y):
    """The op with the norm ("gemma": 1 + w, "plain": w) and the output mode
    ("fp8", "nvfp4", "mxfp8" or None for add + norm alone) chosen, into
    caller-allocated outputs.  MXFP8: ``block_scale`` is the (M, H // 32)
    E8M0 scale buffer and ``scale`` is ignored (may be None)."""
    M, H = x.shape
    with torch.cuda.device(x.device):
        st = _lib.nq_add_rms_norm_quant(
            x.data_ptr(), _ptr(residual), weight.data_ptr(), eps, _ptr(scale), M, H, _DT[x.dtype],
            _NORMS[norm], _MODES[mode], y is not None, _ptr(q), _ptr(block_scale), _ptr(y),
            _stream(x.device))
    _check(st, "nq_add_rms_norm_quant")


def add_rms_norm_quant(x, residual, weight, eps, scale, mode, norm="gemma", write_y=False):
    """Allocating form of add_rms_norm_quant_out: returns (q, block_scale, y)
    as gemma_add_rms_norm_quant does; mode None returns (None, None, y);
    mode "mxfp8" returns E4M3 codes (M, H) and E8M0 scales (M, H // 32)
    (torch.float8_e8m0fnu), both row-major."""
    assert x.dim() == 2 and x.is_contiguous() and x.dtype in _DT and x.is_cuda
    M, H = x.shape
    if mode is None:
        y = torch.empty_like(x)
        if M:
            add_rms_norm_quant_out(x, residual, weight, eps, None, None, norm, None, None, y)
        return None, None, y
    if mode == "nvfp4":
        assert H % 64 == 0
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=x.device)
        block_scale = torch.empty((round_up(M, 128), round_up(H // 16, 4) // 4),
                                  dtype=torch.int32, device=x.device).view(FP8_DTYPE)
    elif mode == "mxfp8":
        assert H % 32 == 0
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=x.device)
        block_scale = torch.empty((M, H // 32), dtype=E8M0_DTYPE, device=x.device)
    else:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=x.device)
        block_scale = scale
    y = torch.empty_like(x) if write_y else None
    if M:
        add_rms_norm_quant_out(x, residual, weight, eps, scale, mode, norm, q,
                               block_scale if mode in ("nvfp4", "mxfp8") else None, y)
    return q, block_scale, y


def gemma_add_rms_norm_mxfp8(x, residual, weight, eps, return_normed=False):
    """Add + Gemma RMSNorm with an MXFP8 output, the single-GPU body of
    ``allreduce_gemma_rms_norm_mxfp8`` (``fused_allreduce_gemma_rms_norm``
    page).  Returns ``(x_q, x_scale, normed, residual)``: E4M3 codes (M, H),
    E8M0 scales (M, H // 32), the normed rows when ``return_normed`` (else
    None), and the residual (updated in place to x + residual; x itself when
    residual is None)."""
    q, s, y = add_rms_norm_quant(x, residual, weight, eps, None, "mxfp8", "gemma", return_normed)
    return q, s, y, (residual if residual is not None else x)


def gemma_add_rms_norm(x, residual, weight, eps):
    """Add + Gemma RMSNorm without quant (residual updated in place); returns y."""
    return add_rms_norm_quant(x, residual, weight, eps, None, None, "gemma", True)[2]


def quant_fp8_static(y, scale, q=None):
    """Standalone static FP8 quant of an activation: E4M3FN(y / scale)."""
    assert y.dim() == 2 and y.is_contiguous() and y.dtype in _DT and y.is_cuda
    M, H = y.shape
    if q is None:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=y.device)
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_fp8_static(y.data_ptr(), scale.data_ptr(), M, H, _DT[y.dtype],
                                          q.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_fp8_static")
    return q


def quant_nvfp4(y, global_scale, q=None, block_scale=None):
    """Standalone NVFP4 quant: packed E2M1 codes and 128x4-tiled E4M3 scales."""
    assert y.dim() == 2 and y.is_contiguous() and y.dtype in _DT and y.is_cuda
    M, H = y.shape
    if q is None:
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=y.device)
    if block_scale is None:
        block_scale = torch.empty((round_up(M, 128), round_up(H // 16, 4) // 4),
                                  dtype=torch.int32, device=y.device).view(FP8_DTYPE)
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_nvfp4(y.data_ptr(), global_scale.data_ptr(), M, H, _DT[y.dtype],
                                     q.data_ptr(), block_scale.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_nvfp4")
    return q, block_scale


def quant_mxfp8(y, q=None, scales=None):
    """Standalone MXFP8 quant: E4M3 codes (M, H) and E8M0 scales (M, H // 32),
    row-major."""
    assert y.dim() == 2 and y.is_contiguous() and y.dtype in _DT and y.is_cuda
    M, H = y.shape
    if q is None:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=y.device)
    if scales is None:
        scales = torch.empty((M, H // 32), dtype=E8M0_DTYPE, device=y.device)
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_mxfp8(y.data_ptr(), M, H, _DT[y.dtype], q.data_ptr(),
                                     scales.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_mxfp8")
    return q, scales


def block_scale_bytes(M, H):
    return _lib.nq_block_scale_bytes(M, H)
