"""Pins of the oracle's add + Gemma RMSNorm steps: torch library routines,
closed forms, exact rational checks and the hand-derived worked examples."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests.golden import read_fixture, num

TORCH = {O.BF16: torch.bfloat16, O.FP16: torch.float16}


def to_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b, fmt):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(TORCH[fmt])


def vals_to_bits(vals, fmt):
    return to_bits(torch.tensor(vals, dtype=torch.float64).to(TORCH[fmt]))


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_residual_add_matches_torch_native_add(fmt):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(64, 512, generator=g) * torch.exp(torch.randn(64, 512, generator=g) * 3))
    r = (torch.randn(64, 512, generator=g) * torch.exp(torch.randn(64, 512, generator=g) * 3))
    x, r = x.to(TORCH[fmt]), r.to(TORCH[fmt])
    ours = O.add_residual(to_bits(x), to_bits(r), fmt)
    assert np.array_equal(ours, to_bits(x + r))


def test_fp8_worked_examples():
    ex, cur = [], None
    for k, v in read_fixture("fp8_worked_examples.txt"):
        if k == "example":
            cur = {}
            ex.append(cur)
        elif k != "quant_case":
            cur[k] = v
    assert len(ex) == 2
    for e in ex:
        fmt = {"bf16": O.BF16, "fp16": O.FP16}[e["dtype"][0]]
        out = O.gemma_add_rms_norm_quant(
            vals_to_bits([[num(t) for t in e["x"]]], fmt),
            vals_to_bits([[num(t) for t in e["residual"]]], fmt),
            vals_to_bits([num(t) for t in e["w"]], fmt),
            num(e["eps"][0]), num(e["scale"][0]), nvfp4=False, write_y=True, fmt=fmt)
        assert [int(v) for v in out["residual"][0]] == [num(t) for t in e["residual_out"]]
        assert [int(v) for v in out["y"][0]] == [num(t) for t in e["y"]]
        assert [int(v) for v in out["q"][0]] == [num(t) for t in e["q"]]


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_constant_rows_closed_form(fmt):
    """eps = 0 and a row of +-2^k: rstd * |h| = 1 exactly, so y = RN(+-(1 + w))."""
    H = 256
    g = torch.Generator().manual_seed(7)
    w = (torch.rand(H, generator=g) * 4 - 2).to(TORCH[fmt])
    k = torch.randint(-8, 8, (6, 1), generator=g).double()
    sign = torch.where(torch.rand(6, H, generator=g) < 0.5, -1.0, 1.0).double()
    h = (sign * torch.pow(2.0, k)).to(TORCH[fmt])
    y = O.gemma_rms_norm(to_bits(h), to_bits(w), 0.0, fmt)
    expect = to_bits((sign * (1.0 + w.double())[None, :]).to(TORCH[fmt]))
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("H", [16, 64, 2048])
def test_eps_adds_to_mean_inside_sqrt(H):
    """A row of 1s with eps = 3: 1/sqrt(1 + 3) = 0.5 exactly, so y = 0.5(1+w).
    (eps outside the root would give 0.25; a sum instead of a mean, or a
    dropped eps, gives other values.)"""
    w = torch.linspace(-0.5, 0.5, H).to(torch.bfloat16)
    h = torch.ones(2, H, dtype=torch.bfloat16)
    y = O.gemma_rms_norm(to_bits(h), to_bits(w), 3.0, O.BF16)
    assert np.array_equal(y, to_bits((0.5 * (1 + w.double())).expand(2, H).to(torch.bfloat16)))


def _near_midpoint(v64, fmt, rel=2.0 ** -22):
    """True where fp64 value v lies within rel of a rounding midpoint of fmt."""
    r = O.round_rne(v64, fmt)
    a = np.abs(v64)
    _, e = np.frexp(np.where(a == 0, 1.0, a))
    ulp = np.ldexp(1.0, np.maximum(e - 1, fmt.emin) - fmt.man_bits)
    frac = np.abs(a - np.abs(r)) / ulp
    return np.abs(frac - 0.5) < rel * np.maximum(a / ulp, 1)


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
@pytest.mark.parametrize("gemma", [False, True])
def test_norm_matches_torch_rms_norm(fmt, gemma):
    """Zero weight is plain RMSNorm; nonzero weight scales by (1 + w).  torch's
    rms_norm in float64 (then * (1 + w)) rounded by torch to the dtype must
    agree except where the float64 value is within 2^-22 (relative) of a
    half-way point: torch rounds float64 -> float32 -> dtype, which lands on
    the tie when the value is within half an fp32 ulp of it."""
    M, H = 32, 1024
    g = torch.Generator().manual_seed(11)
    h = (torch.randn(M, H, generator=g) * 3).to(TORCH[fmt])
    w = (torch.randn(H, generator=g) * 0.3).to(TORCH[fmt]) if gemma else torch.zeros(H, dtype=TORCH[fmt])
    eps = 1e-6
    ours = O.gemma_rms_norm(to_bits(h), to_bits(w), eps, fmt)
    ref64 = torch.nn.functional.rms_norm(h.double(), (H,), eps=float(np.float32(eps))) * (1 + w.double())
    ref = to_bits(ref64.to(TORCH[fmt]))
    diff = ours != ref
    assert not np.any(diff & ~_near_midpoint(ref64.numpy(), fmt))
    assert diff.mean() < 1e-4


def test_weight_minus_one_gives_signed_zero():
    g = torch.Generator().manual_seed(3)
    h = torch.randn(4, 64, generator=g).to(torch.bfloat16)
    w = -torch.ones(64, dtype=torch.bfloat16)
    y = O.gemma_rms_norm(to_bits(h), to_bits(w), 1e-6, O.BF16)
    # (h * rstd) * 0 is +-0 with the sign of h
    expect = np.where((to_bits(h) & 0x8000) != 0, 0x8000, 0).astype(np.uint16)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("k", [-20, -3, 5, 30])
def test_row_scaling_by_power_of_two_leaves_y_unchanged(k):
    g = torch.Generator().manual_seed(13)
    h = torch.randn(8, 320, generator=g).to(torch.bfloat16)
    w = (torch.randn(320, generator=g) * 0.1).to(torch.bfloat16)
    y0 = O.gemma_rms_norm(to_bits(h), to_bits(w), 0.0, O.BF16)
    y1 = O.gemma_rms_norm(to_bits(h * 2.0 ** k), to_bits(w), 0.0, O.BF16)
    assert np.array_equal(y0, y1)


def _exact_within_half_ulp(y_bits, h_bits, w_bits, eps, fmt):
    """Exact rational check that each y is the correctly rounded value of
    h (1+w) / sqrt(mean(h^2) + eps): with v = h(1+w) and d = mean + eps, the
    half-ulp interval [lo, hi] around y must contain v / sqrt(d), i.e.
    lo^2 d <= v^2 <= hi^2 d on the side of y's sign (ties allowed on an edge
    only when y's code is even)."""
    h = [[Fraction(float(v)) for v in row] for row in O.bits_to_f64(h_bits, fmt)]
    w = [Fraction(float(v)) for v in O.bits_to_f64(w_bits, fmt)]
    yv = O.bits_to_f64(y_bits, fmt)
    eps = Fraction(float(np.float32(eps)))
    for i, row in enumerate(h):
        H = len(row)
        d = sum(x * x for x in row) / H + eps
        for j, x in enumerate(row):
            v = x * (1 + w[j])
            y = Fraction(float(yv[i, j]))
            if v == 0:
                assert y == 0
                continue
            assert (y > 0) == (v > 0) or y == 0
            a = abs(y)
            fa = float(a)
            _, e = np.frexp(fa if fa else 1.0)
            ulp = Fraction(2) ** int(max(e - 1, fmt.emin) - fmt.man_bits)
            lo, hi = max(a - ulp / 2, Fraction(0)), a + ulp / 2
            v2 = v * v
            assert lo * lo * d <= v2 <= hi * hi * d, (i, j)


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_y_is_correctly_rounded_exact_arithmetic(fmt):
    g = torch.Generator().manual_seed(17)
    M, H = 3, 16
    x = torch.randn(M, H, generator=g).to(TORCH[fmt])
    r = (torch.randn(M, H, generator=g) * 2).to(TORCH[fmt])
    w = (torch.randn(H, generator=g) * 0.1).to(TORCH[fmt])
    hb = O.add_residual(to_bits(x), to_bits(r), fmt)
    y = O.gemma_rms_norm(hb, to_bits(w), 1e-6, fmt)
    _exact_within_half_ulp(y, hb, to_bits(w), 1e-6, fmt)


def test_no_residual_uses_x_directly():
    g = torch.Generator().manual_seed(19)
    x = torch.randn(4, 128, generator=g).to(torch.bfloat16)
    w = (torch.randn(128, generator=g) * 0.1).to(torch.bfloat16)
    out = O.gemma_add_rms_norm_quant(to_bits(x), None, to_bits(w), 1e-6, 0.02, False, True)
    assert out["residual"] is None
    assert np.array_equal(out["y"], O.gemma_rms_norm(to_bits(x), to_bits(w), 1e-6, O.BF16))


def test_empty_batch():
    for nv in (False, True):
        out = O.gemma_add_rms_norm_quant(np.zeros((0, 64), np.uint16), np.zeros((0, 64), np.uint16),
                                         np.zeros(64, np.uint16), 1e-6, 1.0, nv, True)
        assert out["q"].shape[0] == 0
        if nv:
            assert out["block_scale"].size == 0


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_plain_norm_matches_torch_rms_norm_with_weight(fmt):
    """Plain RMSNorm (scale by w) against torch's rms_norm(weight=w) in
    float64, with the same half-way-point allowance as above."""
    M, H = 16, 768
    g = torch.Generator().manual_seed(23)
    h = (torch.randn(M, H, generator=g) * 2).to(TORCH[fmt])
    w = (torch.randn(H, generator=g) * 0.5 + 1).to(TORCH[fmt])
    ours = O.rms_norm(to_bits(h), to_bits(w), 1e-6, fmt, gemma=False)
    ref64 = torch.nn.functional.rms_norm(h.double(), (H,), weight=w.double(), eps=float(np.float32(1e-6)))
    ref = to_bits(ref64.to(TORCH[fmt]))
    diff = ours != ref
    assert not np.any(diff & ~_near_midpoint(ref64.numpy(), fmt))
    assert diff.mean() < 1e-4


def test_plain_norm_constant_rows_and_gemma_equivalence():
    """Constant rows: plain y = RN(+-w).  And plain(w) == Gemma(w - 1) when
    w - 1 is exact (w a multiple of 2^-7 in [0.5, 2))."""
    H = 128
    g = torch.Generator().manual_seed(29)
    w = (torch.randint(64, 256, (H,), generator=g).double() / 128).to(torch.bfloat16)
    sign = torch.where(torch.rand(3, H, generator=g) < 0.5, -1.0, 1.0).double()
    h = (sign * 4.0).to(torch.bfloat16)
    y = O.rms_norm(to_bits(h), to_bits(w), 0.0, O.BF16, gemma=False)
    assert np.array_equal(y, to_bits((sign * w.double()).to(torch.bfloat16)))
    hr = torch.randn(5, H, generator=g).to(torch.bfloat16)
    wg = (w.double() - 1).to(torch.bfloat16)
    assert torch.equal(wg.double() + 1, w.double())
    assert np.array_equal(O.rms_norm(to_bits(hr), to_bits(w), 1e-6, O.BF16, gemma=False),
                          O.rms_norm(to_bits(hr), to_bits(wg), 1e-6, O.BF16, gemma=True))


def test_no_quant_mode_returns_residual_and_y_only():
    g = torch.Generator().manual_seed(31)
    x = torch.randn(4, 64, generator=g).to(torch.bfloat16)
    r = torch.randn(4, 64, generator=g).to(torch.bfloat16)
    w = (torch.randn(64, generator=g) * 0.1).to(torch.bfloat16)
    out = O.add_rms_norm_quant(to_bits(x), to_bits(r), to_bits(w), 1e-6, None, None)
    assert out["q"] is None and out["block_scale"] is None
    ref = O.gemma_add_rms_norm_quant(to_bits(x), to_bits(r), to_bits(w), 1e-6, 0.1, False, True)
    assert np.array_equal(out["y"], ref["y"]) and np.array_equal(out["residual"], ref["residual"])
