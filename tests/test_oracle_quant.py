"""Pins of the oracle's FP8 and NVFP4 quant steps and of the 128x4 scale
layout: hand-derived worked examples, brute-force nearest-value searches,
error bounds and invariants."""

import numpy as np
import pytest
import torch

import oracle as O
from tests.golden import read_fixture, num
from tests.test_oracle_formats import _brute_nearest_even
from tests.test_oracle_norm import to_bits, vals_to_bits


def test_fp8_quant_cases():
    cases = [[num(t) for t in v] for k, v in read_fixture("fp8_worked_examples.txt") if k == "quant_case"]
    for y, s, code in cases:
        q = O.quant_fp8_static(vals_to_bits([[y]], O.BF16), O.BF16, s)
        assert int(q[0, 0]) == code, (y, s)


@pytest.mark.parametrize("y,s,alt_code", [(0.0888671875, 7.0, 0x07), (0.087890625, 0.9, 0x1D)])
def test_fp8_reciprocal_reading_differs(y, s, alt_code):
    """y * fl32(1/s) gives a different code than y / s on the fixture's
    example C cases, so the tests tell the two readings apart."""
    yf, sf = np.float32(y), np.float32(s)
    alt = O.encode(np.array([float(yf * (np.float32(1) / sf))]), O.E4M3FN)
    assert int(alt[0]) == alt_code


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_fp8_error_bound_and_saturation(fmt):
    """|decode(q) * s - y| <= ulp_E4M3(|y/s|)/2 * s (+ the fp32 division's
    rounding) for |y/s| <= 448; beyond it q is +-448 with y's sign."""
    g = torch.Generator().manual_seed(23)
    y = (torch.randn(64, 512, generator=g) * torch.exp(torch.randn(64, 512, generator=g) * 2))
    yb = to_bits(y.to(torch.bfloat16 if fmt is O.BF16 else torch.float16))
    s = 0.0371
    q = O.quant_fp8_static(yb, fmt, s)
    yv = O.bits_to_f64(yb, fmt)
    dq = O.decode(q, O.E4M3FN)
    v = yv / float(np.float32(s))
    sat = np.abs(v) > 448
    assert np.all(np.abs(dq[sat]) == 448) and np.all(np.sign(dq[sat]) == np.sign(v[sat]))
    a = np.abs(v[~sat])
    _, e = np.frexp(np.where(a == 0, 1, a))
    ulp = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    err = np.abs(dq[~sat] - v[~sat])
    assert np.all(err <= ulp / 2 + np.abs(v[~sat]) * 2.0 ** -23)


def test_fp8_brute_force_nearest():
    g = torch.Generator().manual_seed(29)
    yb = to_bits((torch.randn(16, 4096, generator=g) * 4).to(torch.bfloat16))
    s = np.float32(0.0123)
    q = O.quant_fp8_static(yb, O.BF16, float(s))
    v = O.bits_to_f64(yb, O.BF16).astype(np.float32) / s
    v = np.clip(v, -448, 448).astype(np.float64).reshape(-1)
    assert np.array_equal(q.reshape(-1).astype(np.int64), _brute_nearest_even(v, O.E4M3FN))


def _nvfp4_fixture():
    fx = read_fixture("nvfp4_worked_example.txt")
    d = {}
    for k, v in fx:
        d.setdefault(k, []).extend(v)
    return d


def test_nvfp4_worked_example():
    d = _nvfp4_fixture()
    H = int(num(d["H"][0]))
    w = [num(t) for t in d["w"]]
    assert len(w) == H
    x = vals_to_bits([[num(d["x"][0])] * H], O.BF16)
    r = vals_to_bits([[num(d["residual"][0])] * H], O.BF16)
    out = O.gemma_add_rms_norm_quant(x, r, vals_to_bits(w, O.BF16), num(d["eps"][0]),
                                     num(d["gscale"][0]), nvfp4=True, write_y=True)
    assert np.all(out["residual"] == num(d["residual_out"][0]))
    assert np.array_equal(out["y"][0], vals_to_bits([num(t) for t in d["y"]], O.BF16))
    assert [int(b) for b in out["q"][0]] == [num(t) for t in d["q"]]
    assert [int(b) for b in out["scales"][0]] == [num(t) for t in d["scales"]]
    buf = out["block_scale"]
    assert buf.size == 128 * 4
    assert [int(b) for b in buf[:4]] == [num(t) for t in d["scales"]]
    assert np.all(buf[4:] == 0xA5)


def _gs_fixture():
    d = {}
    for k, v in read_fixture("nvfp4_global_scale_example.txt"):
        d.setdefault(k, []).extend(v)
    y = [num(t) for t in d["y"]]
    assert len(y) == int(num(d["H"][0])) == 64
    return d, y, num(d["gscale"][0])


def test_nvfp4_global_scale_example():
    """Hand-derived NVFP4 quant with gs = 9868951 / 2^15: the block scale is
    fl(gs * fl(a / 6)) rounded to E4M3 and the element multiplier fl(gs /
    sigma) (the fixture's inputs sit on ties where other orders differ)."""
    d, y, gs = _gs_fixture()
    yb = vals_to_bits([y], O.BF16)
    assert np.array_equal(O.bits_to_f64(yb, O.BF16)[0], np.array(y))   # exact bf16 values
    q, S = O.quant_nvfp4(yb, O.BF16, gs)
    assert [int(b) for b in q[0]] == [num(t) for t in d["q"]]
    assert [int(b) for b in S[0]] == [num(t) for t in d["scales"]]
    buf = np.full(128 * 4, 0xA5, np.uint8)
    O.scatter_block_scales(S, 1, 64, buf)
    assert [int(b) for b in buf[:4]] == [num(t) for t in d["scales"]]
    assert np.all(buf[4:] == 0xA5)


def test_nvfp4_global_scale_example_tells_orders_apart():
    """The other plausible fp32 orders, evaluated here directly, give the
    codes the fixture lists as theirs, all different from the fixture's:
    (gs * a) / 6 for the block scale (blocks A and D); gs * fl(1 / sigma),
    1 / fl(sigma / gs) and y / fl(sigma / gs) for the elements (block B)."""
    d, y, gs = _gs_fixture()
    f32 = np.float32
    g = f32(gs)
    yv = np.array(y, dtype=f32).reshape(4, 16)
    a = np.abs(yv).max(axis=1)
    alt_S = O.encode(np.minimum((g * a) / f32(6), f32(448)).astype(np.float64), O.E4M3FN)
    want_alt = [num(t) for t in d["alt_gs_times_a_scales"]]
    assert [int(v) for v in alt_S] == want_alt
    assert want_alt != [num(t) for t in d["scales"]]
    # block A's codes under the alternative block scale
    sig_a = f32(O.decode(np.array([alt_S[0]]), O.E4M3FN)[0])
    ca = O.encode(np.clip(yv[0] * f32(g / sig_a), -6, 6).astype(np.float64), O.E2M1)
    assert [int(ca[2 * k] | (ca[2 * k + 1] << 4)) for k in range(8)] == [num(t) for t in d["alt_gs_times_a_q"]]
    # block B's element codes under each alternative element multiplier
    sig = f32(O.decode(np.array([num(d["scales"][1])]), O.E4M3FN)[0])
    yb_ = yv[1]
    alts = {
        "gs * fl(1/sigma)": yb_ * f32(g * f32(f32(1) / sig)),
        "1 / fl(sigma/gs)": yb_ * f32(f32(1) / f32(sig / g)),
        "y / fl(sigma/gs)": yb_ / f32(sig / g),
    }
    want = [num(t) for t in d["alt_elem_scale_block_b_q"]]
    for name, v in alts.items():
        c = O.encode(np.clip(v.astype(f32), -6, 6).astype(np.float64), O.E2M1)
        got = [int(c[2 * k] | (c[2 * k + 1] << 4)) for k in range(8)]
        assert got == want, name
    assert want != [num(t) for t in d["q"][8:16]]


def test_nvfp4_steps_compose_quant():
    """quant_nvfp4 is its two steps: the block-scale code of each block's
    amax, then the element codes against that scale."""
    yb = _random_y(4, 256, 41, spread=2.0)
    gs = 448 * 6 / 11.0
    q, S = O.quant_nvfp4(yb, O.BF16, gs)
    y = O.bits_to_f64(yb, O.BF16).astype(np.float32).reshape(4, 16, 16)
    assert np.array_equal(S, O.nvfp4_block_scale_codes(np.abs(y).max(axis=2), gs))
    c = O.nvfp4_element_codes(y, S[:, :, None], gs).reshape(4, 256)
    assert np.array_equal(q, (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))


def _random_y(M, H, seed, fmt=O.BF16, spread=1.0):
    g = torch.Generator().manual_seed(seed)
    y = torch.randn(M, H, generator=g) * torch.exp(torch.randn(M, H // 16, 1, generator=g).expand(M, H // 16, 16).reshape(M, H) * spread)
    return to_bits(y.to(torch.bfloat16 if fmt is O.BF16 else torch.float16))


def test_nvfp4_brute_force_scale_and_codes():
    """S is the E4M3 value nearest to gs * (a / 6) (fp32 ops), and each code is
    the E2M1 value nearest to fl32(y * gs / decode(S)) -- both by exhaustive
    search over the code tables."""
    yb = _random_y(8, 1024, 31, spread=2.0)
    gs = np.float32(37.5)
    q, S = O.quant_nvfp4(yb, O.BF16, float(gs))
    y = O.bits_to_f64(yb, O.BF16).astype(np.float32).reshape(8, 64, 16)
    a = np.abs(y).max(axis=2)
    u = np.minimum(gs * (a / np.float32(6)), np.float32(448))
    assert np.array_equal(S.reshape(-1).astype(np.int64), _brute_nearest_even(u.reshape(-1).astype(np.float64), O.E4M3FN))
    sig = O.decode(S, O.E4M3FN).astype(np.float32)
    o = np.where(sig == 0, np.float32(0), gs / np.where(sig == 0, 1, sig)).astype(np.float32)
    v = np.clip(y * o[:, :, None], -6, 6).astype(np.float64).reshape(-1)
    codes = _brute_nearest_even(v, O.E2M1)
    lo = q & 0xF
    hi = q >> 4
    unpacked = np.stack([lo, hi], axis=-1).reshape(-1).astype(np.int64)
    assert np.array_equal(unpacked, codes)


def test_nvfp4_nibble_order_lo_first():
    """Byte k holds element 2k in its low nibble ("lo in the low nibble")."""
    y = np.array([[1.0, 6.0] + [0.0] * 14 + [0.5, -6.0] + [0.0] * 14 + [0.0] * 32])
    q, S = O.quant_nvfp4(vals_to_bits(y, O.BF16), O.BF16, 1.0)
    assert int(q[0, 0]) == 0x72   # codes 2 (1.0) then 7 (6.0)
    assert int(q[0, 8]) == 0xF1   # codes 1 (0.5) then 0xF (-6.0)


def test_nvfp4_block_max_gets_top_code():
    """With u = gs*a/6 in E4M3's normal range, rounding moves the block scale
    by at most 2^-4 relative, so |a * o| is in [5.65, 6.4] and the block's
    largest element always takes magnitude code 7 (6.0)."""
    yb = _random_y(32, 2048, 37, spread=3.0)
    gs = 448 * 6 / 50.0
    q, S = O.quant_nvfp4(yb, O.BF16, gs)
    y = O.bits_to_f64(yb, O.BF16).reshape(32, -1, 16)
    a = np.abs(y).max(axis=2)
    u = np.float32(gs) * (a.astype(np.float32) / np.float32(6))
    normal = (u >= 2.0 ** -6) & (u <= 448)
    codes = np.stack([q & 0xF, q >> 4], -1).reshape(32, -1, 16)
    am = np.abs(y).argmax(axis=2)
    top = np.take_along_axis(codes, am[:, :, None], 2)[:, :, 0] & 0x7
    assert normal.mean() > 0.5
    assert np.all(top[normal] == 7)


def test_nvfp4_dequant_error_bound():
    """Outside saturated blocks, |c * sigma / gs - y| <= half an E2M1 step at
    |y * o| times sigma / gs (plus fp32 rounding of the scale product)."""
    yb = _random_y(16, 1024, 41, spread=1.0)
    gs = np.float32(448 * 6 / 30.0)
    q, S = O.quant_nvfp4(yb, O.BF16, float(gs))
    y = O.bits_to_f64(yb, O.BF16).reshape(16, -1, 16)
    c = np.stack([q & 0xF, q >> 4], -1).reshape(16, -1, 16)
    cv = O.decode(c, O.E2M1)
    sig = O.decode(S, O.E4M3FN)
    ok = sig > 0
    deq = cv * (sig / float(gs))[:, :, None]
    o = float(gs) / np.where(ok, sig, 1)
    t = np.abs(y) * o[:, :, None]
    step = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    bound = (step / 2) * (sig / float(gs))[:, :, None] * (1 + 2.0 ** -20) + np.abs(y) * 2.0 ** -22
    unsat = (t <= 6)
    m = ok[:, :, None] & unsat
    assert m.mean() > 0.9
    assert np.all(np.abs(deq - y)[m] <= bound[m])


def test_nvfp4_zero_and_underflow_blocks():
    y = np.zeros((1, 64))
    y[0, 16:32] = [1e-6] + [0.0] * 15        # u = gs*a/6 underflows E4M3 -> S = 0
    y[0, 32:48] = -1e-7
    q, S = O.quant_nvfp4(vals_to_bits(y, O.BF16), O.BF16, 1.0)
    assert list(S[0, :3]) == [0, 0, 0]
    assert np.all(q[0, :8] == 0)
    assert int(q[0, 8]) == 0x00
    assert np.all(q[0, 16:24] == 0x88)        # negative values keep the sign bit


def test_nvfp4_scale_saturation():
    """u above 448 saturates S to 448 (0x7E); elements then saturate at 6."""
    y = np.full((1, 64), 100.0)
    y[0, 1] = 1.0
    q, S = O.quant_nvfp4(vals_to_bits(y, O.BF16), O.BF16, 448.0)
    assert np.all(S == 0x7E)
    # o = 448/448 = 1: 100 -> 6 (code 7); 1.0 -> code 2
    assert int(q[0, 0]) == 0x27 and np.all(q[0, 1:] == 0x77)


def test_swizzle_fixture_offsets():
    for k, v in read_fixture("swizzle_128x4_offsets.txt"):
        H, m, b, off = (int(num(t)) for t in v)
        assert int(O.swizzle_128x4_offset(m, b, H)) == off, (H, m, b)


@pytest.mark.parametrize("M,H", [(1, 64), (127, 128), (128, 192), (129, 64), (300, 5120)])
def test_swizzle_is_a_bijection_onto_the_padded_buffer(M, H):
    R, C = O.block_scale_buffer_shape(M, H)
    mm, bb = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    off = O.swizzle_128x4_offset(mm, bb, H).reshape(-1)
    assert np.array_equal(np.sort(off), np.arange(R * C))


def test_scatter_leaves_padding_rows_unwritten_and_unswizzles():
    M, H = 130, 128
    rng = np.random.default_rng(0)
    S = rng.integers(0, 0x7E, (M, H // 16)).astype(np.uint8)
    buf = np.full(int(np.prod(O.block_scale_buffer_shape(M, H))), 0xA5, np.uint8)
    O.scatter_block_scales(S, M, H, buf)
    R, C = O.block_scale_buffer_shape(M, H)
    mm, bb = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    off = O.swizzle_128x4_offset(mm, bb, H)
    back = buf[off]
    assert np.array_equal(back[:M], S)
    assert np.all(back[M:] == 0xA5)


# ---------------------------------------------------------------------------
# MXFP8: E4M3FN codes with one E8M0 scale per 32-element block.

def _expand(tokens):
    out = []
    for t in tokens:
        v, _, n = t.partition("*")
        out.extend([num(v)] * (int(n) if n else 1))
    return out


def _mxfp8_fixture():
    fmt, blocks, e2e_w = O.BF16, [], []
    for k, v in read_fixture("mxfp8_worked_examples.txt"):
        if k == "dtype":
            fmt = {"bf16": O.BF16, "fp16": O.FP16}[v[0]]
        elif k == "block":
            blocks.append({"fmt": fmt, "y": _expand(v)})
        elif k in ("codes", "scale"):
            blocks[-1][k] = _expand(v)
        elif k == "e2e_w":
            e2e_w.extend(_expand(v))
    return blocks, e2e_w


def test_mxfp8_worked_blocks():
    blocks, _ = _mxfp8_fixture()
    assert len(blocks) == 10
    for i, b in enumerate(blocks):
        assert len(b["y"]) == 32 and len(b["codes"]) == 32
        yb = vals_to_bits([b["y"]], b["fmt"])
        assert np.array_equal(O.bits_to_f64(yb, b["fmt"])[0], b["y"]), i   # inputs exact
        q, S = O.quant_mxfp8(yb, b["fmt"])
        assert list(q[0]) == b["codes"], (i, list(q[0]))
        assert list(S[0]) == b["scale"], (i, list(S[0]))


def test_mxfp8_worked_example_end_to_end():
    blocks, w = _mxfp8_fixture()
    H = 64
    assert len(w) == H
    x = vals_to_bits([[1.0] * H], O.BF16)
    out = O.add_rms_norm_quant(x, x.copy(), vals_to_bits(w, O.BF16), 0.0, 1.0, "mxfp8")
    assert np.all(out["residual"] == 0x4000)
    assert list(O.bits_to_f64(out["y"], O.BF16)[0]) == blocks[0]["y"] + blocks[1]["y"]
    assert list(out["q"][0]) == blocks[0]["codes"] + blocks[1]["codes"]
    assert list(out["scales"][0]) == blocks[0]["scale"] + blocks[1]["scale"]
    assert out["block_scale"] is out["scales"]


def test_mxfp8_exponent_brute_force():
    """e is the smallest integer >= -127 with amax < 512 * 2^e; for e > -127
    also amax >= 256 * 2^e.  Checked by a linear search with exact ldexp
    comparisons over every bf16 magnitude and every fp16 magnitude."""
    import math
    for fmt in (O.BF16, O.FP16):
        codes = np.arange(0x8000, dtype=np.int64)
        a = O.decode(codes, fmt)
        a = a[np.isfinite(a)]
        e = O.mxfp8_block_exponent(a)
        for ai, ei in zip(a.tolist(), e.tolist()):
            k = -127
            while not ai < math.ldexp(512.0, k):
                k += 1
            assert ei == k, (ai, ei, k)
            if ei > -127:
                assert ai >= math.ldexp(256.0, ei)


def test_mxfp8_codes_brute_force():
    """Each code is the E4M3 value nearest to clamp(y / decode_e8m0(S)), ties
    to the even code, found by exhaustive search over the code table; the
    scale is divided out as a float64 quotient (exact for a power of two)."""
    for fmt in (O.BF16, O.FP16):
        yb = _random_y(8, 1024, 43, fmt=fmt, spread=3.0)
        q, S = O.quant_mxfp8(yb, fmt)
        assert S.shape == (8, 32) and q.shape == (8, 1024)
        y = O.bits_to_f64(yb, fmt).reshape(8, 32, 32)
        v = y / O.decode_e8m0(S)[:, :, None]
        v = np.clip(v, -448, 448).reshape(-1)
        assert np.array_equal(q.reshape(-1).astype(np.int64), _brute_nearest_even(v, O.E4M3FN))


@pytest.mark.parametrize("fmt", [O.BF16, O.FP16])
def test_mxfp8_dequant_error_bound(fmt):
    """decode(q) * 2^e is within half an E4M3 step of y (relative 2^-4 in the
    normal range, 2^-10 * 2^e below it) unless |y| >= 448 * 2^e, where it is
    +-448 * 2^e with y's sign; the block's largest magnitude decodes to
    [256, 448] * 2^e unless the scale is clamped."""
    yb = _random_y(32, 2048, 47, fmt=fmt, spread=4.0)
    q, S = O.quant_mxfp8(yb, fmt)
    y = O.bits_to_f64(yb, fmt).reshape(32, -1, 32)
    sc = O.decode_e8m0(S)[:, :, None]
    dq = O.decode(q, O.E4M3FN).reshape(y.shape) * sc
    sat = np.abs(y) >= 448 * sc
    assert np.all(np.abs(dq[sat]) == (448 * sc * np.ones_like(y))[sat])
    assert np.all(np.sign(dq[sat]) == np.sign(y[sat]))
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * sc)
    assert np.all(np.abs(dq - y)[~sat] <= bound[~sat])
    top = np.abs(dq).max(axis=2)
    unclamped = S > 0
    assert unclamped.mean() > 0.99
    assert np.all((top >= 256 * sc[:, :, 0]) & (top <= 448 * sc[:, :, 0])
                  | ~unclamped)
    assert sat.mean() > 0.0        # the floor rule does saturate some blocks


def test_mxfp8_signed_zero_and_shape_errors():
    y = np.zeros((1, 32))
    y[0, 1] = -0.0
    y[0, 2] = 1.0
    y[0, 3] = -2.0 ** -20             # rounds to -0 on the element grid
    q, S = O.quant_mxfp8(vals_to_bits(y, O.BF16), O.BF16)
    assert int(S[0, 0]) == 127 - 8 and list(q[0, :4]) == [0x00, 0x80, 0x78, 0x80]
    with pytest.raises(ValueError):
        O.quant_mxfp8(vals_to_bits(np.zeros((1, 48)), O.BF16), O.BF16)
    with pytest.raises(ValueError):
        O.add_rms_norm_quant(vals_to_bits(np.ones((1, 48)), O.BF16), None,
                             vals_to_bits(np.zeros(48), O.BF16), 1e-6, 1.0, "mxfp8")
    out = O.add_rms_norm_quant(np.zeros((0, 64), np.uint16), None, vals_to_bits(np.zeros(64), O.BF16),
                               1e-6, 1.0, "mxfp8")
    assert out["q"].shape == (0, 64) and out["scales"].shape == (0, 2)
