"""The op as the unfused chain: add, Gemma RMSNorm, then a standalone quant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the ``fused_norm_quant`` page, ``gemma_add_rms_norm_quant`` (parameter
list, returns, and the wrapper's assertions and output allocation), and the
module docstring there: the fused kernel replaces the Gemma add-RMSNorm
followed by a standalone static-FP8 or NVFP4 quant, computing the codes from
the normed activation rounded to the activation dtype with the same scale
arithmetic, so that the codes equal the unfused chain's.  The
``fused_allreduce_norm_quant`` page (``fused_allreduce_gemma_rms_norm_quant``)
states the same op behind an all-reduce, with fp32 accumulation
(``fp32_acc=True``) and Gemma weight bias 1.

All arrays of activation-dtype values are carried as their 16-bit patterns
(uint16) with a ``Format`` (BF16 or FP16) saying which.

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * the norm reads the rounded sum h (the value written back to residual);
  * eps is added to the mean square inside the square root;
  * weight has x's dtype and the scale factor is (1 + w);
  * y = RN_D(h * rstd * (1 + w)), evaluated here in fp64;
  * FP8: q = E4M3FN_RNE(clamp(fl32(y / s), -448, 448));
  * NVFP4 per 16-element block, all in fp32:
        a = max|y|;  t = a / 6;  u = gs * t;  S = E4M3FN_RNE(min(u, 448));
        o = gs / decode(S)  (0 when S decodes to 0);
        c = E2M1_RNE(clamp(y * o, -6, 6));  byte = c[2k] | c[2k+1] << 4;
  * scale bytes are stored at swizzle_128x4_offset(m, b); rows >= M of the
    padded buffer are never written;
  * MXFP8 (the ``allreduce_gemma_rms_norm_mxfp8`` variant on the
    ``fused_allreduce_gemma_rms_norm`` page, which gives only its outputs'
    types and shapes) per 32-element block, with the OCP MX scale rule:
        a = max|y|;  e = max(floor(log2 a) - 8, -127)  (-127 when a = 0);
        scale code = e + 127 (E8M0);  q = E4M3FN_RNE(clamp(y * 2^-e, +-448)).

Parity (tests/test_oracle_norm.py, tests/test_oracle_quant.py):
  * add_residual: torch's native bf16/fp16 add and the fp32-then-round sum;
  * rms_norm / gemma_rms_norm: closed forms (constant rows, eps placement,
    zero weight = torch's rms_norm, w = -1 gives signed zeros, power-of-two
    row scaling) and an exact rational evaluation of the correctly rounded y;
  * quant_fp8_static: hand-derived examples, two of which tell y / s from
    y * fl(1 / s) apart, a brute-force nearest-code search and the E4M3
    error bound;
  * nvfp4_block_scale_codes / nvfp4_element_codes / quant_nvfp4: a
    hand-derived example with gs = 1 and one with gs = 9868951 / 2^15 whose
    inputs sit on ties where (gs * a) / 6, gs * fl(1 / sigma), 1 /
    fl(sigma / gs) and y / fl(sigma / gs) each give other codes (the
    arithmetic order is a reading of the pages, fixed by this fixture, not
    a parity result against another implementation); brute-force nearest
    codes, the block-max-gets-code-7 invariant, nibble order;
  * quant_mxfp8: ten hand-derived blocks, the block exponent against a
    linear search over every finite bf16 and fp16 magnitude, brute-force
    element codes;
  * swizzle_128x4_offset: hand-derived offsets, bijection, untouched padding.
    The layout itself is named but not defined by the pages: its agreement
    with an outside consumer is parity unpinned.
"""

import numpy as np

from .formats import BF16, FP16, E4M3FN, E2M1, Format, bits_to_f64, f64_to_bits, encode, decode

__all__ = [
    "add_residual", "gemma_rms_norm", "rms_norm", "quant_fp8_static", "quant_nvfp4",
    "nvfp4_block_scale_codes", "nvfp4_element_codes",
    "mxfp8_block_exponent", "quant_mxfp8",
    "swizzle_128x4_offset", "block_scale_buffer_shape", "scatter_block_scales",
    "gemma_add_rms_norm_quant", "add_rms_norm_quant",
]

NVFP4_BLOCK = 16      # elements per NVFP4 block scale
E2M1_MAX = 6.0
E4M3_MAX = 448.0
MX_BLOCK = 32         # elements per MXFP8 scale (scales of shape [M, H // 32])
MX_E4M3_EMAX = 8      # exponent of E4M3FN's largest normal, 448 = 1.75 * 2^8
MX_SCALE_EMIN = -127  # smallest E8M0 exponent


def _check_fmt(fmt: Format):
    if fmt not in (BF16, FP16):
        raise ValueError("activation dtype must be bf16 or fp16")


def add_residual(x_bits, r_bits, fmt: Format) -> np.ndarray:
    """h = RN_D(x + r): the residual after its in-place update.

    The ``residual`` argument of the op on the ``fused_norm_quant`` page is
    overwritten with x + residual (parameter list there).  The sum is taken in float64; when it is not exact
    there, rounding twice (to float64, then to D) still gives the correctly
    rounded sum because 53 >= 2p + 2 for p = 8 (bf16) and p = 11 (fp16).
    """
    _check_fmt(fmt)
    x = bits_to_f64(x_bits, fmt)
    r = bits_to_f64(r_bits, fmt)
    return f64_to_bits(x + r, fmt)


def gemma_rms_norm(h_bits, w_bits, eps: float, fmt: Format) -> np.ndarray:
    """y = RN_D(h / sqrt(mean(h^2) + eps) * (1 + w)), one rounding, fp64.

    ``weight``: the norm scales by (1 + weight) (``fused_norm_quant`` page,
    parameter list; ``weight_bias=1.0 # GemmaRMSNorm-style`` on the
    ``fused_allreduce_gemma_rms_norm`` page).  eps is the RMS-norm epsilon,
    which the kernel receives as an fp32 scalar, so it is first rounded to
    fp32 here.  Row-wise: ``h`` is (M, H), ``w`` is (H,).
    """
    return rms_norm(h_bits, w_bits, eps, fmt, gemma=True)


def rms_norm(h_bits, w_bits, eps: float, fmt: Format, gemma: bool) -> np.ndarray:
    """RMSNorm scaled by (1 + w) (Gemma) or by w (plain RMSNorm, the norm of
    the ``rms_norm_static_fp8_quant`` kernels named on the PR conversation
    page, which multiply the normed value by the weight itself); fp64, one
    rounding."""
    _check_fmt(fmt)
    h = bits_to_f64(h_bits, fmt)
    w = bits_to_f64(w_bits, fmt)
    if h.ndim != 2 or w.shape != (h.shape[1],):
        raise ValueError("h must be (M, H) and w (H,)")
    H = h.shape[1]
    eps64 = float(np.float32(eps))
    mean_sq = np.sum(h * h, axis=1) / H
    rstd = 1.0 / np.sqrt(mean_sq + eps64)
    y = (h * rstd[:, None]) * ((1.0 + w) if gemma else w)[None, :]
    return f64_to_bits(y, fmt)


def quant_fp8_static(y_bits, fmt: Format, scale: float) -> np.ndarray:
    """Static per-tensor FP8: q = E4M3FN_RNE(clamp(fl32(y / scale), +-448)).

    ``scale`` is the static per-tensor input scale of the FP8 mode
    (``fused_norm_quant`` page, parameter list).  The page says the fused
    kernel uses the scale math of the standalone static FP8 quant; dividing
    by the scale is the reading taken here.  Values
    beyond the E4M3FN range saturate to +-448.  Returns uint8 codes, same
    shape as ``y_bits``.
    """
    _check_fmt(fmt)
    y = bits_to_f64(y_bits, fmt).astype(np.float32)        # exact
    s = np.float32(scale)
    with np.errstate(over="ignore"):
        v = y / s                                          # IEEE fp32 divide
    v = np.minimum(np.maximum(v, np.float32(-E4M3_MAX)), np.float32(E4M3_MAX))
    return encode(v.astype(np.float64), E4M3FN)


def nvfp4_block_scale_codes(amax, global_scale) -> np.ndarray:
    """E4M3FN block-scale codes S from block amax values (fp32, >= 0).

    The block's decode scale is amax / 6 (6 is E2M1's largest magnitude),
    mapped into E4M3's range by the global scale gs: u = fl(gs * fl(amax / 6)),
    then S = E4M3FN_RNE(min(u, 448)).  The pages state only that the fused
    kernel uses the standalone NVFP4 quant's scale arithmetic
    (``fused_norm_quant`` page, module docstring); this order of fp32
    operations is the reading taken, and a hand-derived fixture with a
    global scale other than 1 fixes it (the order (gs * amax) / 6 gives
    another code there).
    """
    a = np.asarray(amax, dtype=np.float32)
    gs = np.float32(global_scale)
    t = a / np.float32(E2M1_MAX)                                   # fp32
    with np.errstate(over="ignore"):
        u = gs * t                                                 # fp32
    u = np.minimum(u, np.float32(E4M3_MAX))
    return encode(u.astype(np.float64), E4M3FN).astype(np.uint8)


def nvfp4_element_codes(y, S, global_scale) -> np.ndarray:
    """E2M1 codes (one per element, sign in bit 3) of fp32 values y in a
    block whose E4M3FN scale code is S (broadcast against y).

    The element multiplier is o = fl(gs / decode(S)), 0 for a zero scale;
    each code is E2M1_RNE(clamp(fl(y * o), -6, 6)) (the ``_cvt_e2m1x2``
    helper's ``cvt.rn.satfinite``).  As for the block scale, this order
    (gs divided by the decoded scale, not multiplied by its rounded
    reciprocal) is a reading, fixed by the same fixture.
    """
    y = np.asarray(y, dtype=np.float32)
    gs = np.float32(global_scale)
    sigma = decode(np.asarray(S, dtype=np.uint8), E4M3FN).astype(np.float32)
    o = np.zeros_like(sigma)
    nz = sigma != 0
    o[nz] = gs / sigma[nz]                                         # fp32
    with np.errstate(over="ignore", invalid="ignore"):
        v = y * o                                                  # fp32
    v = np.minimum(np.maximum(v, np.float32(-E2M1_MAX)), np.float32(E2M1_MAX))
    return encode(v.astype(np.float64), E2M1).astype(np.uint8)


def quant_nvfp4(y_bits, fmt: Format, global_scale: float):
    """NVFP4: E2M1 codes with one E4M3FN scale per 16-element block.

    In NVFP4 mode ``scale`` is the global scale, passed as
    ``input_global_scale_inv`` (``fused_norm_quant`` page, parameter list;
    the ``fused_allreduce_norm_quant`` page calls it the inverse of the NVFP4
    global scale) -- read as the multiplier gs that maps a block's decode
    scale amax/6 into the E4M3 range.  E2M1 conversion is
    round-to-nearest-even with saturation (the page's ``_cvt_e2m1x2`` helper
    uses ``cvt.rn.satfinite.e2m1x2.f32``), and each byte holds the
    even-index element in its low nibble (that helper's operand order).
    Per block: ``nvfp4_block_scale_codes`` of its amax, then
    ``nvfp4_element_codes`` of its elements.

    Returns ``(q, S)``: q is (M, H/2) uint8 packed codes; S is the (M, H/16)
    uint8 block-scale codes in row-major order (not yet swizzled).
    """
    _check_fmt(fmt)
    y = bits_to_f64(y_bits, fmt).astype(np.float32)
    M, H = y.shape
    if H % NVFP4_BLOCK:
        raise ValueError("H must be a multiple of 16")
    blk = y.reshape(M, H // NVFP4_BLOCK, NVFP4_BLOCK)
    a = np.max(np.abs(blk), axis=2)                                # exact
    S = nvfp4_block_scale_codes(a, global_scale)
    c = nvfp4_element_codes(blk, S[:, :, None], global_scale).reshape(M, H)
    q = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return q, S


def mxfp8_block_exponent(amax) -> np.ndarray:
    """Shared exponent e of an MX block from its largest magnitude ``amax``.

    The pages give the MXFP8 variant's output types and shapes only
    (``allreduce_gemma_rms_norm_mxfp8``, ``fused_allreduce_gemma_rms_norm``
    page: E4M3 values, one E8M0 scale per 32 values).  Read with the scale
    rule of the OCP Microscaling formats: the block's scale is 2^e with
    e = floor(log2(amax)) minus the exponent of the element format's largest
    normal (8 for E4M3), so the block's largest value lands in [256, 512) on
    the element grid.  e is clamped below at E8M0's smallest exponent -127,
    which also covers an all-zero block.  Exact: frexp gives
    amax = f * 2^k with f in [0.5, 1), so floor(log2(amax)) = k - 1.
    """
    a = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(a)
    e = np.where(a > 0, k.astype(np.int64) - 1 - MX_E4M3_EMAX, MX_SCALE_EMIN)
    return np.maximum(e, MX_SCALE_EMIN).astype(np.int64)


def quant_mxfp8(y_bits, fmt: Format):
    """MXFP8: E4M3FN codes with one E8M0 scale per 32-element block.

    Per block (``mxfp8_block_exponent`` for e): each element is y * 2^-e,
    clamped to +-448 and rounded to nearest even E4M3FN; the block's scale
    code is e + 127.  The scaling by a power of two is exact, so every
    decision here is exact in any precision that holds y * 2^-e down to
    E4M3's half-smallest step.  Values beyond 448 (blocks whose amax has a
    scaled magnitude in [448, 512)) saturate, as the OCP conversion does.

    Returns ``(q, S)``: q is (M, H) uint8 E4M3FN codes and S the (M, H/32)
    uint8 E8M0 codes, both row-major.
    """
    _check_fmt(fmt)
    y = bits_to_f64(y_bits, fmt)
    M, H = y.shape
    if H % MX_BLOCK:
        raise ValueError("H must be a multiple of 32")
    blk = y.reshape(M, H // MX_BLOCK, MX_BLOCK)
    e = mxfp8_block_exponent(np.max(np.abs(blk), axis=2))
    v = np.ldexp(blk, (-e)[:, :, None].astype(np.int32))            # exact
    v = np.minimum(np.maximum(v, -E4M3_MAX), E4M3_MAX)
    q = encode(v, E4M3FN).astype(np.uint8).reshape(M, H)
    return q, (e + 127).astype(np.uint8)


def _round_up(a: int, b: int) -> int:
    return (a + b - 1) // b * b


def block_scale_buffer_shape(M: int, H: int):
    """(round_up(M, 128), round_up(H / 16, 4)) bytes, as the wrapper allocates
    it (``fused_norm_quant`` page, ``gemma_add_rms_norm_quant`` returns and
    allocation)."""
    return (_round_up(M, 128), _round_up(H // NVFP4_BLOCK, 4))


def swizzle_128x4_offset(m, b, H: int):
    """Byte offset of block scale (row m, block b) in the 128x4-tiled layout.

    The pages name the layout (``SWIZZLED_128x4``, and the NVFP4 block scales
    of the op are said to be swizzled 128x4) without spelling it out; this is the 128x4 tiling used for block-scaled
    FP4 GEMM scale operands: 128-row x 4-block tiles of 512 contiguous bytes,
    tiles in row-major order over (m // 128, b // 4), and inside a tile the
    byte for (m, b) at (m % 32) * 16 + ((m % 128) // 32) * 4 + b % 4.
    """
    kp = _round_up(H // NVFP4_BLOCK, 4)
    m = np.asarray(m, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    tile = (m // 128) * (kp // 4) + b // 4
    return tile * 512 + (m % 32) * 16 + ((m % 128) // 32) * 4 + (b % 4)


def scatter_block_scales(S, M: int, H: int, out: np.ndarray) -> np.ndarray:
    """Write row-major scales S (M, H/16) into ``out`` (flat uint8 buffer of
    prod(block_scale_buffer_shape) bytes) at their swizzled offsets.  Bytes
    of rows >= M are left as they were (the op never writes its padding
    rows)."""
    rows, cols = block_scale_buffer_shape(M, H)
    if out.size != rows * cols:
        raise ValueError("wrong block-scale buffer size")
    nb = H // NVFP4_BLOCK
    mm, bb = np.meshgrid(np.arange(M), np.arange(nb), indexing="ij")
    out.reshape(-1)[swizzle_128x4_offset(mm, bb, H).reshape(-1)] = np.asarray(S, np.uint8).reshape(-1)
    return out


def gemma_add_rms_norm_quant(x_bits, residual_bits, weight_bits, eps, scale,
                             nvfp4: bool, write_y: bool = False, fmt: Format = BF16,
                             block_scale_fill: int = 0xA5):
    """The page's op (Gemma norm, FP8 or NVFP4); see add_rms_norm_quant."""
    out = add_rms_norm_quant(x_bits, residual_bits, weight_bits, eps, scale,
                             "nvfp4" if nvfp4 else "fp8", "gemma", fmt, block_scale_fill)
    out["write_y"] = bool(write_y)
    return out


def add_rms_norm_quant(x_bits, residual_bits, weight_bits, eps, scale, mode, norm="gemma",
                       fmt: Format = BF16, block_scale_fill: int = 0xA5):
    """The whole op, as the unfused chain, with the norm ("gemma": 1 + w,
    "plain": w) and the output ("fp8", "nvfp4", "mxfp8", or None: add + norm
    only) chosen.

    Arguments follow ``gemma_add_rms_norm_quant`` on the ``fused_norm_quant``
    page, with x, residual (or None) and weight as 16-bit patterns of
    ``fmt`` and ``scale`` a Python float (fp32 value).  Returns a dict:

      residual : (M, H) uint16, x + residual (None when residual is None)
      q        : FP8 / MXFP8 (M, H) uint8 codes, or NVFP4 (M, H/2) uint8
                 packed codes
      scales   : NVFP4 (M, H/16) row-major E4M3 block-scale codes, MXFP8
                 (M, H/32) E8M0 codes, else None
      block_scale : NVFP4 swizzled buffer (flat uint8, unwritten bytes hold
                 ``block_scale_fill``), MXFP8 the (M, H/32) scales (already
                 row-major), FP8 the scale value itself (``scale`` is
                 ignored for MXFP8)
      y        : (M, H) uint16 normed activation (always computed; the op
                 returns it only when write_y)
    """
    _check_fmt(fmt)
    if mode not in ("fp8", "nvfp4", "mxfp8", None) or norm not in ("gemma", "plain"):
        raise ValueError("mode must be fp8, nvfp4, mxfp8 or None; norm gemma or plain")
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("x must be 2-D")
    M, H = x_bits.shape
    if residual_bits is not None:
        h = add_residual(x_bits, residual_bits, fmt)
    else:
        h = x_bits
    nvfp4 = mode == "nvfp4"
    if nvfp4 and H % 64:
        raise ValueError("NVFP4 needs H % 64 == 0")
    if mode == "mxfp8" and H % MX_BLOCK:
        raise ValueError("MXFP8 needs H % 32 == 0")
    out = {"residual": h if residual_bits is not None else None}
    if M == 0:
        y = np.zeros((0, H), np.uint16)
    else:
        y = rms_norm(h, weight_bits, eps, fmt, gemma=(norm == "gemma"))
    out["y"] = y
    if mode is None:
        out.update(q=None, scales=None, block_scale=None)
    elif nvfp4:
        if M:
            q, S = quant_nvfp4(y, fmt, scale)
        else:
            q, S = np.zeros((0, H // 2), np.uint8), np.zeros((0, H // 16), np.uint8)
        buf = np.full(int(np.prod(block_scale_buffer_shape(M, H))), block_scale_fill, np.uint8)
        scatter_block_scales(S, M, H, buf)
        out.update(q=q, scales=S, block_scale=buf)
    elif mode == "mxfp8":
        if M:
            q, S = quant_mxfp8(y, fmt)
        else:
            q, S = np.zeros((0, H), np.uint8), np.zeros((0, H // MX_BLOCK), np.uint8)
        out.update(q=q, scales=S, block_scale=S)
    else:
        q = quant_fp8_static(y, fmt, scale) if M else np.zeros((0, H), np.uint8)
        out.update(q=q, scales=None, block_scale=float(np.float32(scale)))
    return out
