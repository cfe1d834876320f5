"""Number formats of the op, written out from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formats used by the op:

* bf16 and fp16 -- the activation dtypes (the ``x`` argument of
  ``gemma_add_rms_norm_quant`` on the ``fused_norm_quant`` page may be
  either).  IEEE-style: an all-ones exponent field is Inf/NaN.
* E4M3FN -- the FP8 code of the static per-tensor mode and of the NVFP4 block
  scales (``FP8_DTYPE`` / ``current_platform.fp8_dtype()`` on the
  ``fused_norm_quant`` and ``fused_allreduce_norm_quant`` pages).  Read as the
  OCP "FN" variant: bias 7, no infinities, only S.1111.111 is NaN, largest
  finite value 448.
* E2M1 -- the NVFP4 element code (``_cvt_e2m1x2`` on the ``fused_norm_quant``
  page): bias 1, one mantissa bit, no Inf/NaN, largest value 6.
* E8M0 -- the MXFP8 block-scale code (the scales, one per 32 values and
  stored row by row, that ``allreduce_gemma_rms_norm_mxfp8`` returns on the
  ``fused_allreduce_gemma_rms_norm`` page).  Read as the scale type of the OCP Microscaling (MX) formats: an
  unsigned 8-bit exponent with bias 127 and nothing else, value
  2**(code - 127); no sign, no zero, code 255 is NaN.

Rounding (``round_rne``): the nearest value on the format's grid, ties to the
value whose code has an even mantissa field (round-to-nearest-even), with
gradual underflow below the smallest normal.  Written generically: a value
``a`` with leading-bit exponent ``E`` (clamped below at the format's minimum
normal exponent) sits on the grid of multiples of ``2**(E - mantissa_bits)``;
``numpy.rint`` rounds the (exact, power-of-two scaled) quotient half-to-even.
An even multiple is exactly an even mantissa field, including the step into
the next binade.

Parity: pinned by tests/test_oracle_formats.py -- decode tables against
torch's CPU float8_e4m3fn/bfloat16/float16 casts, the E2M1 table against the
golden list of its eight magnitudes, and every encoder against (a) torch's CPU
casts and (b) a brute-force nearest-value search, over every tie and
tie-neighbour of the fp32 inputs that matter plus random inputs; the E8M0
table against torch's CPU float8_e8m0fnu.
"""

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Format:
    name: str
    exp_bits: int
    man_bits: int
    bias: int
    ieee_specials: bool   # all-ones exponent encodes Inf/NaN (bf16, fp16)
    fn_nan_only: bool     # only S.1..1.1..1 is NaN, no Inf (E4M3FN)

    @property
    def bits(self) -> int:
        return 1 + self.exp_bits + self.man_bits

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal value."""
        return 1 - self.bias

    @property
    def max_finite(self) -> float:
        t = decode_table(self)
        return float(np.max(t[np.isfinite(t)]))


BF16 = Format("bf16", 8, 7, 127, True, False)
FP16 = Format("fp16", 5, 10, 15, True, False)
E4M3FN = Format("e4m3fn", 4, 3, 7, False, True)
E2M1 = Format("e2m1", 2, 1, 1, False, False)

_TABLES = {}


def decode(codes, fmt: Format) -> np.ndarray:
    """Value of each code (float64), from the sign/exponent/mantissa fields."""
    c = np.asarray(codes).astype(np.int64) & ((1 << fmt.bits) - 1)
    s = (c >> (fmt.bits - 1)) & 1
    e = (c >> fmt.man_bits) & ((1 << fmt.exp_bits) - 1)
    m = c & ((1 << fmt.man_bits) - 1)
    frac = m.astype(np.float64) / float(1 << fmt.man_bits)
    sub = np.ldexp(frac, fmt.emin)                      # 0.m * 2^emin
    nrm = np.ldexp(1.0 + frac, (e - fmt.bias).astype(np.int32))  # 1.m * 2^(e-bias)
    mag = np.where(e == 0, sub, nrm)
    emax_field = (1 << fmt.exp_bits) - 1
    if fmt.ieee_specials:
        mag = np.where(e == emax_field, np.where(m == 0, np.inf, np.nan), mag)
    if fmt.fn_nan_only:
        mag = np.where((e == emax_field) & (m == (1 << fmt.man_bits) - 1), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def decode_e8m0(codes) -> np.ndarray:
    """Value of each E8M0 code (float64): 2**(code - 127), NaN for 255."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.ldexp(1.0, (c - 127).astype(np.int32)))


def decode_table(fmt: Format) -> np.ndarray:
    """Values of all 2**bits codes, indexed by code."""
    if fmt.name not in _TABLES:
        _TABLES[fmt.name] = decode(np.arange(1 << fmt.bits), fmt)
    return _TABLES[fmt.name]


def _positive_finite(fmt: Format):
    """(values, codes) of the non-negative finite codes, ascending."""
    t = decode_table(fmt)
    half = 1 << (fmt.bits - 1)
    vals = t[:half]
    ok = np.isfinite(vals)
    codes = np.arange(half)[ok]
    vals = vals[ok]
    assert np.all(np.diff(vals) > 0)
    return vals, codes


def round_rne(v, fmt: Format) -> np.ndarray:
    """Round float64 values to the format's grid, nearest, ties to even.

    No saturation and no overflow handling: the result may lie above the
    format's largest finite value (callers clamp first for the saturating
    FP8/FP4 encoders; ``f64_to_bits`` maps overflow of bf16/fp16 to Inf).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                 # a = f * 2**e, f in [0.5, 1)
    lead = np.maximum(e - 1, fmt.emin)  # exponent of the leading bit, >= emin
    ulp_exp = (lead - fmt.man_bits).astype(np.int32)
    q = np.rint(np.ldexp(a, -ulp_exp))  # exact scaling; rint = half-to-even
    r = np.ldexp(q, ulp_exp)
    return np.copysign(r, v)


def encode(v, fmt: Format) -> np.ndarray:
    """Code (integer of ``fmt.bits`` bits) of the RNE rounding of ``v``.

    ``v`` must round to a finite value of the format (clamp first for E4M3FN
    and E2M1).  The sign bit follows the sign of ``v``, so -0 and negative
    values that round to zero give the negative-zero code.
    """
    v = np.asarray(v, dtype=np.float64)
    r = round_rne(v, fmt)
    vals, codes = _positive_finite(fmt)
    a = np.abs(r)
    idx = np.searchsorted(vals, a)
    idx_c = np.minimum(idx, len(vals) - 1)
    if not np.all(vals[idx_c] == a):
        bad = a[vals[idx_c] != a]
        raise ValueError(f"{fmt.name}: value(s) outside the finite range: {bad[:4]}")
    code = codes[idx_c]
    sign = np.signbit(r).astype(np.int64) << (fmt.bits - 1)
    return (code | sign).astype(np.uint16 if fmt.bits > 8 else np.uint8)


def f64_to_bits(v, fmt: Format) -> np.ndarray:
    """bf16/fp16 bits of the RNE rounding of float64 ``v``; overflow -> Inf."""
    assert fmt.ieee_specials
    v = np.asarray(v, dtype=np.float64)
    r = round_rne(v, fmt)
    inf_code = ((1 << fmt.exp_bits) - 1) << fmt.man_bits
    over = np.abs(r) > fmt.max_finite
    r_fin = np.where(over, 0.0, r)
    code = encode(r_fin, fmt).astype(np.int64)
    sign = np.signbit(r).astype(np.int64) << (fmt.bits - 1)
    code = np.where(over, inf_code | sign, code)
    return code.astype(np.uint16)


def bits_to_f64(bits, fmt: Format) -> np.ndarray:
    """Exact float64 value of bf16/fp16 bit patterns."""
    return decode(np.asarray(bits).astype(np.int64), fmt)
