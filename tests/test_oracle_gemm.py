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


# ---- NVFP4 consumer -------------------------------------------------------

_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _frac_e2m1(c):
    return (-1 if c & 8 else 1) * _E2M1[c & 7]


def _nvfp4_operand(rng, rows, K, scale_codes):
    """Random packed E2M1 codes and a 128x4-tiled scale buffer whose block
    scales are drawn from ``scale_codes``; also returns the row-major scale
    codes."""
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.int64).astype(np.uint8)
    S = np.asarray(scale_codes, np.uint8)[rng.integers(0, len(scale_codes), size=(rows, K // 16))]
    buf = np.zeros(int(np.prod(O.block_scale_buffer_shape(rows, K))), np.uint8)
    O.scatter_block_scales(S, rows, K, buf)
    return q, S, buf


def test_nvfp4_gemm_exact_rational():
    rng = np.random.default_rng(7)
    M, N, K = 3, 5, 128
    codes = [0x30, 0x38, 0x39, 0x3C, 0x44, 0x2A, 0x51]          # 0.5, 1, 1.125, 1.5, 3, 0.3125, 36
    aq, aS, abuf = _nvfp4_operand(rng, M, K, codes)
    bq, bS, bbuf = _nvfp4_operand(rng, N, K, codes)
    ga, gb = 2.5, 0.75
    exact, bits = O.gemm_nvfp4(aq, abuf, ga, bq, bbuf, gb, M, N, K)
    for m in range(M):
        for n in range(N):
            ref = Fraction(0)
            for k in range(K):
                ca = (int(aq[m, k // 2]) >> (4 * (k % 2))) & 15
                cb = (int(bq[n, k // 2]) >> (4 * (k % 2))) & 15
                ref += _frac_e2m1(ca) * _frac_e4m3(aS[m, k // 16]) * _frac_e2m1(cb) * _frac_e4m3(bS[n, k // 16])
            ref /= Fraction(ga) * Fraction(gb)
            assert abs(exact[m, n] - float(ref)) <= 1e-14 * max(1.0, abs(float(ref)))
    assert bits.dtype == np.uint16 and bits.shape == (M, N)


def test_nvfp4_element_order_and_scale_placement():
    """Byte j of a row holds element 2 j in its low nibble; the scale of
    (row m, block b) sits at the 128x4-tiled offset, checked at hand-computed
    offsets of a 130-row, 8-block (K = 128) buffer."""
    M, K = 130, 128
    # a: row 33 has a single 1.0 (code 2) at element 81 (byte 40, high nibble),
    # row 129 a single 1.0 at element 32 (byte 16, low nibble); b: all ones.
    aq = np.zeros((M, K // 2), np.uint8)
    aq[33, 40] = 0x20
    aq[129, 16] = 0x02
    abuf = np.zeros(256 * 8, np.uint8)
    # element 81 is in block 5 of row 33: tile 1 (rows 0..127, blocks 4..7),
    # 512 + (33 % 32) * 16 + (33 // 32) * 4 + 5 % 4 = 533
    abuf[533] = 0x40                                   # 2.0
    # element 32 is in block 2 of row 129: tile 2, 1024 + 1 * 16 + 0 + 2 = 1042
    abuf[1042] = 0x48                                  # 4.0
    bq = np.full((1, K // 2), 0x22, np.uint8)          # every element 1.0
    bbuf = np.full(128 * 8, 0x38, np.uint8)            # every scale 1.0
    exact, _ = O.gemm_nvfp4(aq, abuf, 1.0, bq, bbuf, 1.0, M, 1, K)
    want = np.zeros((M, 1))
    want[33, 0] = 2.0
    want[129, 0] = 4.0
    assert np.array_equal(exact, want)
    # moving row 33's code to the low nibble (element 80) keeps block 5
    aq[33, 40] = 0x02
    assert O.gemm_nvfp4(aq, abuf, 1.0, bq, bbuf, 1.0, M, 1, K)[0][33, 0] == 2.0
    # a B operand that is zero except element 81 selects the high nibble
    bq2 = np.zeros((1, K // 2), np.uint8)
    bq2[0, 40] = 0x20
    aq[33, 40] = 0x20
    assert O.gemm_nvfp4(aq, abuf, 1.0, bq2, bbuf, 1.0, M, 1, K)[0][33, 0] == 2.0
    aq[33, 40] = 0x02
    assert O.gemm_nvfp4(aq, abuf, 1.0, bq2, bbuf, 1.0, M, 1, K)[0][33, 0] == 0.0


def test_nvfp4_closed_form_and_global_scale_law():
    M, N, K = 2, 3, 256
    aq = np.full((M, K // 2), 0x22, np.uint8)          # 1.0 everywhere
    bq = np.full((N, K // 2), 0x33, np.uint8)          # 1.5 everywhere
    abuf = np.full(128 * 16, 0x38, np.uint8)           # scale 1.0
    bbuf = np.full(128 * 16, 0x40, np.uint8)           # scale 2.0
    exact, bits = O.gemm_nvfp4(aq, abuf, 1.0, bq, bbuf, 1.0, M, N, K)
    assert np.all(exact == K * 1.0 * 3.0)
    assert np.all(O.bits_to_f64(bits, O.BF16) == 768.0)
    half, _ = O.gemm_nvfp4(aq, abuf, 2.0, bq, bbuf, 1.0, M, N, K)
    third, _ = O.gemm_nvfp4(aq, abuf, 1.0, bq, bbuf, 3.0, M, N, K)
    assert np.all(half == exact / 2) and np.allclose(third, exact / 3, rtol=1e-15)


def test_nvfp4_gemm_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.dequant_nvfp4(np.zeros((2, 40), np.uint8), np.zeros(128 * 8, np.uint8), 1.0, 2, 80)
    with pytest.raises(ValueError):
        O.dequant_nvfp4(np.zeros((2, 32), np.uint8), np.zeros(128 * 8, np.uint8), 1.0, 2, 128)
