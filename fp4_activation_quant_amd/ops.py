"""PyTorch-facing entry points of the HIP library.

PyTorch supplies device memory and the current stream; every step of the op
runs in the library (``_lib`` only marshals pointers).  The public call
``gemma_add_rms_norm_quant`` keeps the interface of the op on the
``fused_norm_quant`` page -- the same arguments, the same output tuple and
output shapes -- so callers of that op can switch to it unchanged; the other
functions expose the library's variants (plain norm, no quant, MXFP8) and
the standalone quant kernels of the unfused chain.
"""

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.NQ_BF16, torch.float16: _lib.NQ_FP16}
_MODES = {"fp8": _lib.NQ_MODE_FP8_STATIC, "nvfp4": _lib.NQ_MODE_NVFP4, "mxfp8": _lib.NQ_MODE_MXFP8,
          None: _lib.NQ_MODE_NONE}
_NORMS = {"gemma": _lib.NQ_NORM_GEMMA, "plain": _lib.NQ_NORM_PLAIN}
FP8_DTYPE = torch.float8_e4m3fn
E8M0_DTYPE = torch.float8_e8m0fnu


def round_up(a, b):
    return -(-a // b) * b


def _check(status, what):
    if status != _lib.NQ_OK:
        raise _lib.NqError(status, what)


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _validate(x, residual, weight, scale):
    _require(x.is_cuda and x.dim() == 2 and x.is_contiguous(), "x: contiguous 2-D device tensor")
    _require(x.dtype in _DT, "x: bfloat16 or float16")
    if residual is not None:
        _require(residual.shape == x.shape and residual.dtype == x.dtype and
                 residual.device == x.device and residual.is_contiguous(),
                 "residual: contiguous, same shape, dtype and device as x")
    _require(weight.shape == (x.shape[1],) and weight.dtype == x.dtype and weight.is_contiguous()
             and weight.device == x.device, "weight: contiguous (H,) of x's dtype, on x's device")
    if scale is not None:
        _require(scale.numel() == 1 and scale.dtype == torch.float32 and scale.device == x.device,
                 "scale: one float32 on x's device")


def _outputs(M, H, mode, dev, scale):
    """(q, block_scale) buffers for an output mode; the FP8 "block scale" is
    the caller's scale tensor itself."""
    if mode == "nvfp4":
        _require(H % 64 == 0, "NVFP4 needs H % 64 == 0")
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
        # 128x4-tiled E4M3 scales, rows padded to 128 and scale columns to 4;
        # the padding rows are never written.
        bs = torch.empty((round_up(M, 128), round_up(H // 16, 4)), dtype=torch.uint8,
                         device=dev).view(FP8_DTYPE)
        return q, bs
    if mode == "mxfp8":
        _require(H % 32 == 0, "MXFP8 needs H % 32 == 0")
        return (torch.empty((M, H), dtype=FP8_DTYPE, device=dev),
                torch.empty((M, H // 32), dtype=E8M0_DTYPE, device=dev))
    return torch.empty((M, H), dtype=FP8_DTYPE, device=dev), scale


def _validate_out(x, mode, q, block_scale, y):
    """Caller-supplied outputs: on x's device, contiguous, large enough, of
    one-byte (codes, scales) or x's (y) elements; alignment is the library's
    business (unaligned views take its scalar path)."""
    M, H = x.shape
    dev = x.device
    if mode is not None:
        _buf(q, "q", dev, nbytes=M * (H // 2) if mode == "nvfp4" else M * H, itemsize=1)
    if mode == "nvfp4":
        _buf(block_scale, "block_scale", dev, nbytes=_lib.nq_block_scale_bytes(M, H))
    elif mode == "mxfp8":
        _buf(block_scale, "block_scale", dev, nbytes=M * (H // 32), itemsize=1)
    if y is not None:
        _buf(y, "y", dev, nbytes=M * H * x.element_size(), dtype=x.dtype)


def add_rms_norm_quant_out(x, residual, weight, eps, scale, mode, norm, q, block_scale, y):
    """One launch of the op into caller-allocated buffers; no allocation.
    Every tensor is checked (device, contiguity, size, element type) before
    its pointer goes to the library.

    ``norm``: "gemma" (scale by 1 + w) or "plain" (by w).  ``mode``: "fp8"
    (static per-tensor, ``scale`` = the dequant scale), "nvfp4" (``scale`` =
    global scale, ``block_scale`` = the 128x4-tiled buffer), "mxfp8"
    (``block_scale`` = (M, H // 32) E8M0 scales, ``scale`` ignored) or None
    (add + norm only; ``y`` required).  ``y`` None: the normed activation is
    not written."""
    _validate(x, residual, weight, scale if mode in ("fp8", "nvfp4") else None)
    _validate_out(x, mode, q, block_scale, y)
    M, H = x.shape
    with torch.cuda.device(x.device):
        st = _lib.nq_add_rms_norm_quant(
            x.data_ptr(), _ptr(residual), weight.data_ptr(), eps, _ptr(scale), M, H, _DT[x.dtype],
            _NORMS[norm], _MODES[mode], y is not None, _ptr(q), _ptr(block_scale), _ptr(y),
            _stream(x.device))
    _check(st, "nq_add_rms_norm_quant")


def gemma_add_rms_norm_quant_out(x, residual, weight, eps, scale, nvfp4, q, block_scale, y):
    """The page's op (Gemma norm, FP8 or NVFP4) into caller-allocated buffers,
    through the library's own entry point for it (same checks as
    ``add_rms_norm_quant_out``)."""
    _validate(x, residual, weight, scale)
    _validate_out(x, "nvfp4" if nvfp4 else "fp8", q, block_scale, y)
    M, H = x.shape
    with torch.cuda.device(x.device):
        st = _lib.nq_gemma_add_rms_norm_quant(
            x.data_ptr(), _ptr(residual), weight.data_ptr(), eps, scale.data_ptr(), M, H,
            _DT[x.dtype], _lib.NQ_MODE_NVFP4 if nvfp4 else _lib.NQ_MODE_FP8_STATIC, y is not None,
            q.data_ptr(), _ptr(block_scale), _ptr(y), _stream(x.device))
    _check(st, "nq_gemma_add_rms_norm_quant")


def add_rms_norm_quant(x, residual, weight, eps, scale, mode, norm="gemma", write_y=False):
    """Allocating form of ``add_rms_norm_quant_out``.  Returns
    ``(q, block_scale, y)``: codes, scales (FP8: ``scale`` itself), and the
    normed activation when ``write_y`` (always for mode None, which returns
    ``(None, None, y)``).  ``residual`` (or None) is updated in place."""
    _validate(x, residual, weight, scale if mode in ("fp8", "nvfp4") else None)
    M, H = x.shape
    if mode is None:
        y = torch.empty_like(x)
        if M:
            add_rms_norm_quant_out(x, residual, weight, eps, None, None, norm, None, None, y)
        return None, None, y
    q, bs = _outputs(M, H, mode, x.device, scale)
    y = torch.empty_like(x) if write_y else None
    if M:
        add_rms_norm_quant_out(x, residual, weight, eps, scale, mode, norm, q,
                               bs if mode != "fp8" else None, y)
    return q, bs, y


def gemma_add_rms_norm_quant(x, residual, weight, eps, scale, nvfp4, write_y=False):
    """Fused residual add + Gemma RMSNorm + input quant for the next linear.

    ``x`` (M, H) bf16 or fp16 is only read.  ``residual`` (same shape and
    dtype, or None) receives x + residual.  The norm multiplies by
    (1 + ``weight``).  ``scale`` is one float32 on the device: the static
    FP8 dequant scale, or with ``nvfp4`` the NVFP4 global scale.  Returns
    ``(q, block_scale, y)``:

    * FP8: q (M, H) float8_e4m3fn, block_scale = ``scale``;
    * NVFP4 (H % 64 == 0): q (M, H // 2) uint8, two E2M1 codes per byte;
      block_scale (round_up(M, 128), round_up(H // 16, 4)) float8_e4m3fn in
      the 128x4-tiled layout, padding rows untouched;
    * y: the normed activation in x's dtype when ``write_y``, else None.
    """
    _validate(x, residual, weight, scale)
    M, H = x.shape
    q, bs = _outputs(M, H, "nvfp4" if nvfp4 else "fp8", x.device, scale)
    y = torch.empty_like(x) if write_y else None
    if M:
        gemma_add_rms_norm_quant_out(x, residual, weight, eps, scale, nvfp4, q,
                                     bs if nvfp4 else None, y)
    return q, bs, y


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


def _validate_y(y):
    _require(y.is_cuda and y.dim() == 2 and y.is_contiguous() and y.dtype in _DT,
             "y: contiguous 2-D bfloat16/float16 device tensor")


def _buf(t, name, dev, shape=None, nbytes=None, itemsize=None, dtype=None):
    """A caller-supplied tensor the library reads or writes by pointer:
    contiguous, on ``dev``, and of the stated shape / size / element type."""
    _require(isinstance(t, torch.Tensor) and t.is_cuda and t.device == dev and t.is_contiguous(),
             f"{name}: contiguous tensor on {dev}")
    if shape is not None:
        _require(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(shape)}, got {tuple(t.shape)}")
    if nbytes is not None:
        _require(t.numel() * t.element_size() >= nbytes, f"{name}: at least {nbytes} bytes")
    if itemsize is not None:
        _require(t.element_size() == itemsize, f"{name}: {itemsize}-byte elements")
    if dtype is not None:
        _require(t.dtype == dtype, f"{name}: {dtype}")


def _scalar(t, name, dev):
    _buf(t, name, dev, dtype=torch.float32)
    _require(t.numel() == 1, f"{name}: one float32")


def quant_fp8_static(y, scale, q=None):
    """Standalone static FP8 quant of an activation: E4M3FN(y / scale)."""
    _validate_y(y)
    M, H = y.shape
    _scalar(scale, "scale", y.device)
    if q is None:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=y.device)
    _buf(q, "q", y.device, shape=(M, H), itemsize=1)
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_fp8_static(y.data_ptr(), scale.data_ptr(), M, H, _DT[y.dtype],
                                          q.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_fp8_static")
    return q


def quant_nvfp4(y, global_scale, q=None, block_scale=None):
    """Standalone NVFP4 quant: packed E2M1 codes and 128x4-tiled E4M3 scales."""
    _validate_y(y)
    M, H = y.shape
    _require(H % 16 == 0, "the standalone NVFP4 quant needs H % 16 == 0")
    _scalar(global_scale, "global_scale", y.device)
    if q is None:
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=y.device)
    if block_scale is None:
        block_scale = torch.empty((round_up(M, 128), round_up(H // 16, 4)), dtype=torch.uint8,
                                  device=y.device).view(FP8_DTYPE)
    _buf(q, "q", y.device, shape=(M, H // 2), itemsize=1)
    _buf(block_scale, "block_scale", y.device, nbytes=_lib.nq_block_scale_bytes(M, H))
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_nvfp4(y.data_ptr(), global_scale.data_ptr(), M, H, _DT[y.dtype],
                                     q.data_ptr(), block_scale.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_nvfp4")
    return q, block_scale


def quant_mxfp8(y, q=None, scales=None):
    """Standalone MXFP8 quant: E4M3 codes (M, H) and E8M0 scales (M, H // 32),
    row-major."""
    _validate_y(y)
    M, H = y.shape
    _require(H % 32 == 0, "MXFP8 needs H % 32 == 0")
    if q is None:
        q = torch.empty((M, H), dtype=FP8_DTYPE, device=y.device)
    if scales is None:
        scales = torch.empty((M, H // 32), dtype=E8M0_DTYPE, device=y.device)
    _buf(q, "q", y.device, shape=(M, H), itemsize=1)
    _buf(scales, "scales", y.device, shape=(M, H // 32), itemsize=1)
    if M:
        with torch.cuda.device(y.device):
            st = _lib.nq_quant_mxfp8(y.data_ptr(), M, H, _DT[y.dtype], q.data_ptr(),
                                     scales.data_ptr(), _stream(y.device))
        _check(st, "nq_quant_mxfp8")
    return q, scales


def _validate_codes(q, name, dev=None):
    _require(q.is_cuda and q.dim() == 2 and q.is_contiguous() and q.element_size() == 1,
             f"{name}: contiguous 2-D one-byte device tensor")
    _require(dev is None or q.device == dev, f"{name}: on {dev}")


def _gemm_out(out, M, N, dev):
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _buf(out, "out", dev, shape=(M, N), dtype=torch.bfloat16)
    return out


def gemm_mxfp8(a, a_scales, b, b_scales, out=None):
    """The consumer linear on an MXFP8 activation: out (M, N) bf16 =
    dq(a) @ dq(b)^T, with a (M, K) / b (N, K) E4M3 codes and (rows, K // 32)
    E8M0 scales, all row-major (the MXFP8 mode's outputs, and a weight in the
    same format)."""
    _validate_codes(a, "a")
    _validate_codes(b, "b", a.device)
    M, K = a.shape
    N = b.shape[0]
    _require(b.shape[1] == K and K % 32 == 0, "b: (N, K) with the same K; K % 32 == 0")
    _buf(a_scales, "a_scales", a.device, shape=(M, K // 32), itemsize=1)
    _buf(b_scales, "b_scales", a.device, shape=(N, K // 32), itemsize=1)
    out = _gemm_out(out, M, N, a.device)
    with torch.cuda.device(a.device):
        st = _lib.nq_gemm_mxfp8(a.data_ptr(), a_scales.data_ptr(), b.data_ptr(), b_scales.data_ptr(),
                                M, N, K, out.data_ptr(), _stream(a.device))
    _check(st, "nq_gemm_mxfp8")
    return out


def gemm_fp8_static(a, a_scale, b, b_scale, out=None):
    """The consumer linear on a static-FP8 activation: out (M, N) bf16 =
    (a * a_scale) @ (b * b_scale)^T, scales one float32 each on the device."""
    _validate_codes(a, "a")
    _validate_codes(b, "b", a.device)
    M, K = a.shape
    N = b.shape[0]
    _require(b.shape[1] == K and K % 32 == 0, "b: (N, K) with the same K; K % 32 == 0")
    _scalar(a_scale, "a_scale", a.device)
    _scalar(b_scale, "b_scale", a.device)
    out = _gemm_out(out, M, N, a.device)
    with torch.cuda.device(a.device):
        st = _lib.nq_gemm_fp8_static(a.data_ptr(), a_scale.data_ptr(), b.data_ptr(), b_scale.data_ptr(),
                                     M, N, K, out.data_ptr(), _stream(a.device))
    _check(st, "nq_gemm_fp8_static")
    return out


def gemma_add_rms_norm_quant_gemm_fp8_out(x, residual, residual_out, weight, eps, scale, b, b_scale, q, y,
                                          out):
    """A decode step: the op in static FP8 mode (codes into ``q``, ``y`` if
    given, x + ``residual`` into ``residual_out``) and the consumer linear
    ``out`` (M, N) bf16 = dq(q) @ dq(b)^T of the FP8 weight ``b`` (N, H)
    with its float32 scale; one launch up to 3 rows, the op and the decode
    GEMM as two launches from 4.  For 1 <= M <= 8 and H in {1024, 2048,
    4096}; other shapes raise (call the op and ``gemm_fp8_static``).  The
    residual is not updated in place (``residual_out`` is its own buffer)."""
    _validate(x, residual, weight, scale)
    M, H = x.shape
    dev = x.device
    if residual is not None:
        _buf(residual_out, "residual_out", dev, shape=(M, H), dtype=x.dtype)
    _validate_codes(b, "b", dev)
    _require(b.shape[1] == H, "b: (N, H)")
    _scalar(b_scale, "b_scale", dev)
    _buf(q, "q", dev, nbytes=M * H, itemsize=1)
    if y is not None:
        _buf(y, "y", dev, nbytes=M * H * x.element_size(), dtype=x.dtype)
    N = b.shape[0]
    _buf(out, "out", dev, shape=(M, N), dtype=torch.bfloat16)
    with torch.cuda.device(dev):
        st = _lib.nq_gemma_add_rms_norm_quant_gemm_fp8(
            x.data_ptr(), _ptr(residual), _ptr(residual_out) if residual is not None else 0, weight.data_ptr(),
            eps, scale.data_ptr(), M, H, _DT[x.dtype], y is not None, q.data_ptr(), _ptr(y), b.data_ptr(),
            b_scale.data_ptr(), N, out.data_ptr(), _stream(dev))
    _check(st, "nq_gemma_add_rms_norm_quant_gemm_fp8")


def gemm_nvfp4(a, a_block_scale, a_global_scale, b, b_block_scale, b_global_scale, out=None):
    """The consumer linear on an NVFP4 activation: out (M, N) bf16 =
    dq(a) @ dq(b)^T, with a (M, K // 2) / b (N, K // 2) packed E2M1 codes,
    their 128x4-tiled E4M3 block-scale buffers (the NVFP4 mode's outputs, and
    a weight in the same format) and one float32 global scale each on the
    device (dq = code * block scale / global scale)."""
    _validate_codes(a, "a")
    _validate_codes(b, "b", a.device)
    M, K = a.shape[0], 2 * a.shape[1]
    N = b.shape[0]
    _require(b.shape[1] == K // 2 and K % 64 == 0, "b: (N, K // 2) with the same K; K % 64 == 0")
    _buf(a_block_scale, "a_block_scale", a.device, nbytes=_lib.nq_block_scale_bytes(M, K))
    _buf(b_block_scale, "b_block_scale", a.device, nbytes=_lib.nq_block_scale_bytes(N, K))
    _scalar(a_global_scale, "a_global_scale", a.device)
    _scalar(b_global_scale, "b_global_scale", a.device)
    out = _gemm_out(out, M, N, a.device)
    with torch.cuda.device(a.device):
        st = _lib.nq_gemm_nvfp4(a.data_ptr(), a_block_scale.data_ptr(), a_global_scale.data_ptr(), b.data_ptr(),
                                b_block_scale.data_ptr(), b_global_scale.data_ptr(), M, N, K, out.data_ptr(),
                                _stream(a.device))
    _check(st, "nq_gemm_nvfp4")
    return out


def block_scale_bytes(M, H):
    return _lib.nq_block_scale_bytes(M, H)
