"""Pins of the oracle's number formats against torch's CPU casts, brute-force
nearest-value searches and the hand-derived E2M1 fixture."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.golden import read_fixture, num


def _tie_heavy_f32(exp_lo=-140, exp_hi=130, low_zero_bits=12, seed=0, n_random=200_000):
    """fp32 values whose low ``low_zero_bits`` mantissa bits are zero, over a
    band of exponents, with their +-1 ulp neighbours and random values.

    Every round-to-nearest tie of a conversion to a format with <= 11 stored
    mantissa bits (bf16, fp16, E4M3, E2M1) has its low 12 bits zero, so the
    set holds every tie in the band together with the values just either side.
    """
    hi = np.arange(1 << (23 - low_zero_bits), dtype=np.uint32) << low_zero_bits
    exps = np.arange(max(exp_lo + 127, 0), min(exp_hi + 127, 254) + 1, dtype=np.uint32)
    base = (exps[:, None] << 23 | hi[None, :]).reshape(-1)
    vals = [base, base + 1, base - 1]
    rng = np.random.default_rng(seed)
    vals.append(rng.integers(0, 0x7F800000, n_random, dtype=np.uint32))
    u = np.concatenate(vals)
    u = u[(u & 0x7F800000) != 0x7F800000]
    u = np.concatenate([u, u | 0x80000000])
    return u.view(np.float32)


def test_bf16_fp16_decode_match_torch():
    codes = np.arange(1 << 16, dtype=np.int64)
    for fmt, tdt in ((O.BF16, torch.bfloat16), (O.FP16, torch.float16)):
        ours = O.decode(codes, fmt)
        ref = torch.from_numpy(codes.astype(np.int16)).view(tdt).double().numpy()
        assert np.array_equal(ours, ref, equal_nan=True), fmt.name


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.int64)
    ours = O.decode(codes, O.E4M3FN)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    assert O.E4M3FN.max_finite == 448.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.int64)
    ours = O.decode_e8m0(codes)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(ours, ref, equal_nan=True)
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127
    assert np.isnan(ours[255])


def test_e2m1_decode_matches_fixture():
    fx = dict((k, v) for k, v in read_fixture("e2m1_format.txt") if k == "values")
    vals = [num(t) for t in fx["values"]]
    t = O.decode_table(O.E2M1)
    assert list(t[:8]) == vals
    assert list(-t[8:]) == vals and all(np.signbit(t[8:]))


def test_e2m1_encoder_fixture_cases():
    cases = [(num(v[0]), num(v[1])) for k, v in read_fixture("e2m1_format.txt") if k == "case"]
    v = np.array([a for a, _ in cases], np.float32)
    v = np.minimum(np.maximum(v, np.float32(-6)), np.float32(6))
    got = O.encode(v.astype(np.float64), O.E2M1)
    assert [int(g) for g in got] == [c for _, c in cases]


def _brute_nearest_even(v, fmt):
    """Nearest finite value by exhaustive search over the code table; ties go
    to the code whose mantissa field is even.  Returns codes."""
    t = O.decode_table(fmt)
    half = 1 << (fmt.bits - 1)
    codes = np.arange(half)
    vals = t[:half]
    ok = np.isfinite(vals)
    codes, vals = codes[ok], vals[ok]
    a = np.abs(v)[:, None]
    d = np.abs(a - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = (codes & 1) == 0
    pick_even = cand & even[None, :]
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
    assert np.all(cand.sum(axis=1) <= 2)
    return codes[idx] | (np.signbit(v).astype(np.int64) << (fmt.bits - 1))


@pytest.mark.parametrize("fmt,lim", [(O.E4M3FN, 448.0), (O.E2M1, 6.0)])
def test_small_encoders_vs_brute_force(fmt, lim):
    v = _tie_heavy_f32(exp_lo=-14 if fmt is O.E4M3FN else -4,
                       exp_hi=10 if fmt is O.E4M3FN else 4, low_zero_bits=14, n_random=20_000)
    v = np.minimum(np.maximum(v, np.float32(-lim)), np.float32(lim)).astype(np.float64)
    for chunk in np.array_split(v, 16):
        assert np.array_equal(O.encode(chunk, fmt).astype(np.int64), _brute_nearest_even(chunk, fmt))


def test_e4m3_encoder_vs_torch_cast():
    """Saturating E4M3FN encoding of fp32 (clamp to +-448, then RNE) against
    torch's CPU float8_e4m3fn cast, over every tie and tie-neighbour of all
    fp32 exponents plus random values."""
    v = _tie_heavy_f32()
    v = np.minimum(np.maximum(v, np.float32(-448)), np.float32(448))
    ours = O.encode(v.astype(np.float64), O.E4M3FN)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("fmt,tdt", [(O.BF16, torch.bfloat16), (O.FP16, torch.float16)])
def test_half_rounding_of_f32_vs_torch(fmt, tdt):
    """RNE of fp32 to bf16/fp16 (incl. subnormals and overflow to Inf) against
    torch's CPU casts."""
    v = _tie_heavy_f32()
    ours = O.f64_to_bits(v.astype(np.float64), fmt)
    ref = torch.from_numpy(v).to(tdt).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_direct_rounding_of_f64_is_single(fmt):
    """fp64 values a hair above/below a half-way point must round away from
    it; rounding through fp32 first would land on the tie and go to even."""
    rng = np.random.default_rng(1)
    lo_codes = rng.integers(0x0400, 0x7000 if fmt is O.BF16 else 0x7800, 5000)
    lo = O.decode(lo_codes, fmt)
    hi = O.decode(lo_codes + 1, fmt)
    mid = (lo + hi) / 2                       # exact in fp64
    up = mid * (1 + 2.0 ** -40)
    dn = mid * (1 - 2.0 ** -40)
    assert np.array_equal(O.f64_to_bits(up, fmt), (lo_codes + 1).astype(np.uint16))
    assert np.array_equal(O.f64_to_bits(dn, fmt), lo_codes.astype(np.uint16))
    tie = O.f64_to_bits(mid, fmt).astype(np.int64)
    assert np.all(tie % 2 == 0) and np.all((tie == lo_codes) | (tie == lo_codes + 1))
    neg = O.f64_to_bits(-up, fmt).astype(np.int64)
    assert np.array_equal(neg, (lo_codes + 1) | 0x8000)


def test_negative_zero_codes():
    assert int(O.encode(np.array([-0.0]), O.E4M3FN)[0]) == 0x80
    assert int(O.encode(np.array([-1e-9]), O.E4M3FN)[0]) == 0x80
    assert int(O.encode(np.array([-0.0]), O.E2M1)[0]) == 0x8
    assert int(O.f64_to_bits(np.array([-0.0]), O.BF16)[0]) == 0x8000
