"""Pins of the consumer-GEMM oracle: exact rational evaluation on small
inputs, closed forms, scale laws and operand orientation."""

from fractions import Fraction

import numpy as np
import pytest

import oracle as O


def _codes(rng, shape):
    """Random finite E4M3FN codes (NaN patterns excluded)."""
    c = rng.integers(0, 256, size=shape, dtype=np.int64)
    c = np.where((c & 0x7F) == 0x7F, c - 1, c)
    return c.astype(np.uint8)


def _frac_e4m3(c):
    """Exact value of an E4M3FN code from its fields (independent of the
    oracle's decode)."""
    c = int(c)
    sgn = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 0xF, c & 7
    v = Fraction(m, 8) * Fraction(1, 2 ** 6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return sgn * v


def test_mxfp8_gemm_exact_rational():
    rng = np.random.default_rng(5)
    M, N, K = 3, 4, 96
    aq, bq = _codes(rng, (M, K)), _codes(rng, (N, K))
    as_ = rng.integers(110, 140, size=(M, K // 32)).astype(np.uint8)
    bs = rng.integers(110, 140, size=(N, K // 32)).astype(np.uint8)
    exact, bits = O.gemm_mxfp8(aq, as_, bq, bs)
    for m in range(M):
        for n in range(N):
            ref = sum(_frac_e4m3(aq[m, k]) * _frac_e4m3(bq[n, k])
                      * Fraction(2) ** (int(as_[m, k // 32]) + int(bs[n, k // 32]) - 254) for k in range(K))
            assert exact[m, n] == float(ref) or abs(exact[m, n] - float(ref)) <= 1e-15 * abs(float(ref))
    assert bits.dtype == np.uint16 and bits.shape == (M, N)


def test_fp8_static_gemm_exact_rational():
    rng = np.random.default_rng(6)
    M, N, K = 2, 3, 64
    aq, bq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa, sb = 0.0137, 2.5
    exact, _ = O.gemm_fp8_static(aq, sa, bq, sb)
    fa, fb = Fraction(float(np.float32(sa))), Fraction(float(np.float32(sb)))
    for m in range(M):
        for n in range(N):
            ref = sum(_frac_e4m3(aq[m, k]) * fa * _frac_e4m3(bq[n, k]) * fb for k in range(K))
            assert abs(exact[m, n] - float(ref)) <= 1e-14 * float(sum(
                abs(_frac_e4m3(aq[m, k]) * fa * _frac_e4m3(bq[n, k]) * fb) for k in range(K)))


def test_ones_closed_form_and_block_scale_law():
    K = 128
    a = np.full((2, K), 0x38, np.uint8)            # 1.0
    b = np.full((3, K), 0x38, np.uint8)
    sa = np.full((2, K // 32), 127, np.uint8)       # 2^0
    sb = np.full((3, K // 32), 127, np.uint8)
    exact, bits = O.gemm_mxfp8(a, sa, b, sb)
    assert np.all(exact == K) and np.all(bits == 0x4300)  # bf16 128.0
    sa2 = sa.copy()
    sa2[1, 2] = 128                                 # row 1, block 2 doubled
    exact2, _ = O.gemm_mxfp8(a, sa2, b, sb)
    assert np.all(exact2[0] == K) and np.all(exact2[1] == K + 32)
    sb2 = sb.copy()
    sb2[2, 0] = 125                                 # column 2, block 0 quartered
    exact3, _ = O.gemm_mxfp8(a, sa, b, sb2)
    assert np.all(exact3[:, 2] == K - 32 + 8) and np.all(exact3[:, :2] == K)


def test_operand_orientation():
    """A is (M, K) and B is (N, K), both K-contiguous: a single product lands
    at [m, n] only when the k indices agree."""
    K = 64
    a = np.zeros((3, K), np.uint8)
    b = np.zeros((4, K), np.uint8)
    a[1, 5] = 0x40                                  # 2.0
    b[2, 5] = 0x44                                  # 3.0
    s3, s4 = np.full((3, 2), 127, np.uint8), np.full((4, 2), 127, np.uint8)
    exact, _ = O.gemm_mxfp8(a, s3, b, s4)
    want = np.zeros((3, 4))
    want[1, 2] = 6.0
    assert np.array_equal(exact, want)
    b2 = np.zeros_like(b)
    b2[2, 6] = 0x44
    assert np.all(O.gemm_mxfp8(a, s3, b2, s4)[0] == 0)


def test_static_scales_multiply():
    rng = np.random.default_rng(9)
    aq, bq = _codes(rng, (4, 64)), _codes(rng, (5, 64))
    e1, _ = O.gemm_fp8_static(aq, 1.0, bq, 1.0)
    e2, _ = O.gemm_fp8_static(aq, 0.5, bq, 4.0)
    assert np.array_equal(e2, e1 * 2.0)


def test_bad_scale_shapes_raise():
    with pytest.raises(ValueError):
        O.dequant_mxfp8(np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8))
    with pytest.raises(ValueError):
        O.dequant_mxfp8(np.zeros((2, 64), np.uint8), np.zeros((2, 3), np.uint8))
