"""Exactness claims behind the kernels' shortened divisions, checked in exact
rational arithmetic on the CPU (no GPU, no oracle): each claim is about an
instruction sequence on IEEE binary32 with round-to-nearest-even, so the
sequence is evaluated step by step with Fractions and every step rounded by
rn32 below.  The GPU probe tests then compare the kernels' own results with
the oracle."""

from fractions import Fraction as F

import numpy as np


def rn32(x: F) -> F:
    """x rounded to the nearest binary32 value, ties to even (no overflow)."""
    if x == 0:
        return F(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    ulp = F(2) ** (max(e, -126) - 23)
    q, r = divmod(a, ulp)
    if 2 * r > ulp or (2 * r == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def _nonneg_16bit_values():
    """Every non-negative finite value an fp16 or a bf16 holds."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    b = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    return sorted(set(h.tolist()) | set(b.tolist()))


def test_rn32_against_numpy():
    rng = np.random.default_rng(5)
    for v in rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000):
        assert rn32(F(float(v))) == F(float(np.float32(v)))


def test_div6_one_correction_exact_for_16bit_amax():
    """NVFP4 block scale: fl32(a / 6) for every amax a that a bf16 or an fp16
    holds is q0 + (a - 6 q0) r with r = fl(1/6), q0 = fl(a r), the remainder
    and the final step each one FMA (one rounding)."""
    r = rn32(F(1, 6))
    assert r == F(float(np.float32(1.0) / np.float32(6.0)))
    vals = _nonneg_16bit_values()
    assert len(vals) == 60032
    wrong = []
    for v in vals:
        a = F(v)
        q0 = rn32(a * r)
        e = rn32(q0 * 6 - a)
        q1 = rn32(q0 - e * r)
        if q1 != rn32(a / 6):
            wrong.append(v)
    assert not wrong, wrong[:5]


def test_div6_needs_the_correction():
    """The plain product alone is not enough (so the test above would catch
    a dropped correction): fl(a r) differs from fl32(a / 6) for many a."""
    r = rn32(F(1, 6))
    vals = _nonneg_16bit_values()
    assert sum(rn32(F(v) * r) != rn32(F(v) / 6) for v in vals[::7]) > 1000


def _finite_16bit(fmt):
    if fmt == "fp16":
        v = np.arange(0, 1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32)
    else:
        v = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    return v[np.isfinite(v)]


def test_fp8_division_in_fp64_is_fl32():
    """Static FP8: the kernels form fl32(y / s) as RN32(RN64(y * RN64(1/s)))
    for y that a bf16 or an fp16 holds.  Against numpy's correctly rounded
    fp32 division, every finite 16-bit y of both formats, 300 scales over 80
    binades plus amax / 448 scales of short amax values (whose quotients
    land on fp32 values that are E4M3 rounding ties): equal wherever the
    quotient is a normal fp32, and below 2^-10 (the code +-0) with the same
    sign where it is not."""
    rng = np.random.default_rng(23)
    scales = list(2.0 ** rng.uniform(-40, 40, 300))
    scales += [a / 448 for a in (7.0625, 6.96875, 6.1875, 25.125, 7.46484375, 1.0, 3.0, 113.0, 0.75)]
    for fmt in ("fp16", "bf16"):
        y = _finite_16bit(fmt)
        for s in scales:
            s32 = np.float32(s)
            with np.errstate(over="ignore"):       # infinite quotients on both sides
                want = y / s32
                got = (y.astype(np.float64) * (1.0 / np.float64(s32))).astype(np.float32)
            normal = np.abs(want) >= np.float32(2.0 ** -126)
            assert np.array_equal(got[normal], want[normal]), (fmt, float(s32))
            sub = ~normal
            assert np.all(np.abs(got[sub]) < 2.0 ** -10)
            assert np.array_equal(np.signbit(got[sub]), np.signbit(want[sub]))
