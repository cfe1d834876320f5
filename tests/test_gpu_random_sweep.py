"""GPU parity over seeded random sweeps, through the C ABI.

The op: output mode (static FP8, NVFP4, MXFP8, none), activation dtype,
residual or not, write_y or not, Gemma or plain norm, misaligned views, and
shapes drawn across every launch form (several rows per wave for H <= 512,
one workgroup per row, the looping launch at 4096 < H < 6144 with 2048 <=
M <= 16384, the element-wise path for H % 16 != 0 or unaligned pointers),
with special values injected into some cases (zero norm factors, rows with
h = 0, rows scaled up to saturate or down into subnormals).  Every case is
compared with the oracle on every row, to the same bars as the fixed
workloads (tests/parity.py).

The standalone quant kernels: random shapes and dynamic ranges, codes and
scales bit-exact against the oracle's quant steps.  The consumer GEMMs:
random shapes across their kernels, on operands whose every partial sum is
exact in fp32, so the bf16 result must equal the oracle's bit for bit."""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib, ops
from tests import parity as P

pytestmark = pytest.mark.gpu

SEED = 20261202
NCASES = 96
MAX_ELEMS = 15_000_000


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _draw_cases():
    rng = np.random.default_rng(SEED)
    cases = []
    for i in range(NCASES):
        mode = ["fp8", "nvfp4", "mxfp8", "none"][int(rng.integers(4))]
        dt = [torch.bfloat16, torch.float16][int(rng.integers(2))]
        res = bool(rng.integers(2))
        wy = bool(rng.integers(2)) or mode == "none"
        norm = "plain" if rng.random() < 0.25 else "gemma"
        unit = {"nvfp4": 64, "mxfp8": 32}.get(mode, 16)
        kind = rng.random()
        if kind < 0.2:                                   # several rows per wave
            H = unit * int(rng.integers(1, 512 // unit + 1))
        elif kind < 0.45:                                # the looping launch's range
            H = unit * int(rng.integers(4096 // unit + 1, 6144 // unit))
        elif kind < 0.85:                                # one workgroup per row
            H = unit * int(rng.integers(512 // unit + 1, 12288 // unit + 1))
        else:                                            # H % 16 != 0: element-wise path (FP8, none)
            H = int(rng.integers(1, 6000)) if mode in ("fp8", "none") else unit * int(rng.integers(1, 64))
        if 4096 < H < 6144 and rng.random() < 0.7:
            M = int(rng.integers(2048, 2400))
        else:
            M = int(np.exp(rng.uniform(0.0, np.log(3000.0))))
        M = max(1, min(M, MAX_ELEMS // H))
        misalign = rng.random() < 0.1
        xs, rs, ws = float(rng.uniform(0.1, 4.0)), float(rng.uniform(0.1, 4.0)), float(rng.uniform(0.0, 0.5))
        # y is about the normalised activation times (1 + w): a few units at most
        spread = float(np.exp(rng.uniform(np.log(0.5), np.log(2.0))))
        scale = {"fp8": 4.0 / 448.0 * spread, "nvfp4": 448.0 * 6.0 / 4.0 * spread}.get(mode, 1.0)
        special = [k for k, pk in (("zero_factor", 0.3), ("zero_h", 0.2), ("big_row", 0.2), ("tiny_row", 0.1))
                   if rng.random() < pk]
        cases.append(dict(i=i, mode=mode, dt=dt, res=res, wy=wy, norm=norm, M=M, H=H, misalign=misalign,
                          xs=xs, rs=rs, ws=ws, scale=scale, special=special, seed=SEED + 7919 * i))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{i}-{mode}-{M}x{H}".format(**c))
def test_random_case_matches_oracle(case):
    c = case
    print(f"random case {c['i']}: {c['mode']} {c['dt']} M={c['M']} H={c['H']} res={c['res']} "
          f"write_y={c['wy']} norm={c['norm']} misalign={c['misalign']} scale={c['scale']:.6g} "
          f"special={c['special']}", flush=True)
    g = torch.Generator().manual_seed(c["seed"])
    M, H, dt = c["M"], c["H"], c["dt"]
    x = torch.randn(M, H, generator=g) * c["xs"]
    r = torch.randn(M, H, generator=g) * c["rs"] if c["res"] else None
    w = torch.randn(H, generator=g) * c["ws"]
    sp = c["special"]
    if "zero_factor" in sp:                              # norm factor exactly 0 in every 7th column
        w[::7] = -1.0 if c["norm"] == "gemma" else 0.0
    k = int(torch.randint(M, (1,), generator=g))
    if "big_row" in sp:                                  # saturating codes (x100 keeps fp16 finite)
        x[k] *= 100.0 if dt == torch.float16 else 1e4
        if r is not None:
            r[k] *= 100.0 if dt == torch.float16 else 1e4
    if "tiny_row" in sp:                                 # values down in the subnormals
        x[(k + 1) % M] *= 1e-6
        if r is not None:
            r[(k + 1) % M] *= 1e-6
    x, w = x.to(dt), w.to(dt)
    r = r.to(dt) if r is not None else None
    if "zero_h" in sp and r is not None:                 # h = x + r = +0 across one row
        r[(k + 2) % M] = -x[(k + 2) % M]
    mode = c["mode"]
    gpu = P.run_gpu(x, r.clone() if r is not None else None, w, 1e-6, c["scale"], mode == "nvfp4", c["wy"],
                    misalign=c["misalign"], norm=c["norm"], quant=mode != "none", mxfp8=mode == "mxfp8")
    rep = P.check(P.compare(gpu, x, r, w, 1e-6, c["scale"], P.all_rows(M)))
    print(rep, flush=True)


def _draw_quant_cases(n=32):
    rng = np.random.default_rng(SEED + 1)
    out = []
    for i in range(n):
        dt = [torch.bfloat16, torch.float16][int(rng.integers(2))]
        kind = rng.random()
        H = (16 * int(rng.integers(1, 640)) if kind < 0.6 else 32 * int(rng.integers(1, 320)) if kind < 0.85
             else int(rng.integers(1, 6000)))
        M = max(1, min(int(np.exp(rng.uniform(0.0, np.log(3000.0)))), 8_000_000 // H))
        out.append(dict(i=i, dt=dt, M=M, H=H, seed=SEED + 104729 * i, s=float(np.exp(rng.uniform(-9, 2))),
                        gs=float(448 * 6 * np.exp(rng.uniform(-3, 3)))))
    return out


@pytest.mark.parametrize("case", _draw_quant_cases(), ids=lambda c: "{i}-{M}x{H}".format(**c))
def test_random_standalone_quant_matches_oracle_exactly(case):
    """The quant step alone is a function of y: static FP8 codes (any H),
    NVFP4 codes and 128x4-tiled scales (H % 16 == 0; padding bytes
    untouched) and MXFP8 codes and scales (H % 32 == 0) must equal the
    oracle's bit for bit."""
    c = case
    print(f"random quant case {c['i']}: {c['dt']} M={c['M']} H={c['H']} s={c['s']:.4g} gs={c['gs']:.4g}",
          flush=True)
    g = torch.Generator().manual_seed(c["seed"])
    M, H, dt = c["M"], c["H"], c["dt"]
    y = (torch.randn(M, H, generator=g) * torch.exp(2 * torch.randn(M, 1, generator=g))).to(dt)
    y[0, :: 5] = 0.0
    y[-1, 1:: 5] = -0.0
    dev = torch.device("cuda")
    yd, yb, fmt = y.to(dev), P.bits16(y), P.FMT[dt]
    s = torch.tensor([c["s"]], dtype=torch.float32, device=dev)
    q = ops.quant_fp8_static(yd, s)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), O.quant_fp8_static(yb, fmt, float(s.item())))
    if H % 16 == 0:
        gs = torch.tensor([c["gs"]], dtype=torch.float32, device=dev)
        nb = ops.block_scale_bytes(M, H)
        bs = torch.full((nb,), P.SENTINEL, dtype=torch.uint8, device=dev)
        qn, _ = ops.quant_nvfp4(yd, gs, block_scale=bs)
        qr, S = O.quant_nvfp4(yb, fmt, float(gs.item()))
        assert np.array_equal(qn.cpu().numpy(), qr)
        want = np.full(nb, P.SENTINEL, np.uint8)
        O.scatter_block_scales(S, M, H, want)
        assert np.array_equal(bs.cpu().numpy(), want)
    if H % 32 == 0:
        qm, sm = ops.quant_mxfp8(yd)
        qr, sr = O.quant_mxfp8(yb, fmt)
        assert np.array_equal(qm.view(torch.uint8).cpu().numpy(), qr)
        assert np.array_equal(sm.view(torch.uint8).cpu().numpy().reshape(M, H // 32), sr)


# E4M3 codes of +-{0.5, 1, 1.5, 2, 3, 4} and zero: products of two are
# multiples of 2^-2 below 16 (with block scales 2^-1 .. 2^1, multiples of
# 2^-4 below 64), so every partial sum up to K = 16384 is exact in fp32.
_E4M3_SMALL = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0xB0, 0xB8, 0xBC, 0xC0, 0xC4, 0xC8], np.uint8)


def _draw_gemm_cases(n=40):
    rng = np.random.default_rng(SEED + 2)
    out = []
    for i in range(n):
        fmt = ["mxfp8", "fp8", "nvfp4"][int(rng.integers(3))]
        kind = rng.random()
        M = (int(rng.integers(1, 9)) if kind < 0.25 else int(rng.integers(9, 257)) if kind < 0.6
             else int(rng.integers(257, 2300)))
        N = int(np.exp(rng.uniform(np.log(8), np.log(6000))))
        unit = 64 if fmt == "nvfp4" else 32
        K = unit * int(rng.integers(1, 16384 // unit + 1)) if rng.random() < 0.4 else \
            512 * int(rng.integers(1, 17))
        while M * N * K > 3e9:
            K = max(unit, K // 2 // unit * unit)
        out.append(dict(i=i, fmt=fmt, M=M, N=N, K=K, seed=SEED + 15485863 * i))
    return out


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("case", _draw_gemm_cases(), ids=lambda c: "{i}-{fmt}-{M}x{N}x{K}".format(**c))
def test_random_gemm_matches_oracle_exactly(case):
    c = case
    print(f"random gemm case {c['i']}: {c['fmt']} M={c['M']} N={c['N']} K={c['K']}", flush=True)
    rng = np.random.default_rng(c["seed"])
    M, N, K = c["M"], c["N"], c["K"]
    out = torch.full((M * N * 2 + P.GUARD,), P.SENTINEL, dtype=torch.uint8, device="cuda")
    o = out[:M * N * 2].view(torch.bfloat16).view(M, N)
    f32 = lambda v: torch.tensor([v], dtype=torch.float32, device="cuda")
    if c["fmt"] == "nvfp4":
        # codes within +-2, block scales 0.5 .. 1.5, power-of-two global
        # scales: every partial sum is a multiple of 2^-8 below 2^24 units
        nib = np.array([0, 1, 2, 3, 4, 9, 10, 11, 12], np.uint8)
        sc = np.array([0x30, 0x38, 0x39, 0x3C], np.uint8)

        def operand(rows):
            n = nib[rng.integers(0, len(nib), size=(rows, K))]
            q = (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)
            S = sc[rng.integers(0, len(sc), size=(rows, K // 16))]
            buf = rng.integers(0, 0x7F, size=int(np.prod(O.block_scale_buffer_shape(rows, K)))).astype(np.uint8)
            O.scatter_block_scales(S, rows, K, buf)
            return q, buf
        aq, ab = operand(M)
        bq, bb = operand(N)
        ga, gb = [(1.0, 1.0), (2.0, 0.5), (0.25, 4.0)][int(rng.integers(3))]
        ops.gemm_nvfp4(_dev(aq), _dev(ab), f32(ga), _dev(bq), _dev(bb), f32(gb), out=o)
        _, want = O.gemm_nvfp4(aq, ab, ga, bq, bb, gb, M, N, K)
    else:
        aq = _E4M3_SMALL[rng.integers(0, len(_E4M3_SMALL), size=(M, K))]
        bq = _E4M3_SMALL[rng.integers(0, len(_E4M3_SMALL), size=(N, K))]
        if c["fmt"] == "mxfp8":
            as_ = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
            bs = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
            ops.gemm_mxfp8(_dev(aq), _dev(as_), _dev(bq), _dev(bs), out=o)
            _, want = O.gemm_mxfp8(aq, as_, bq, bs)
        else:
            ops.gemm_fp8_static(_dev(aq), f32(0.25), _dev(bq), f32(2.0), out=o)
            _, want = O.gemm_fp8_static(aq, 0.25, bq, 2.0)
    torch.cuda.synchronize()
    assert bool((out[M * N * 2:] == P.SENTINEL).all()), "wrote past the output"
    got = P.bits16(o)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], want[bad][:5])


def _draw_decode_cases(n=24):
    rng = np.random.default_rng(SEED + 3)
    return [dict(i=i, dt=[torch.bfloat16, torch.float16][int(rng.integers(2))], M=int(rng.integers(1, 9)),
                 H=[1024, 2048, 4096][int(rng.integers(3))], N=int(np.exp(rng.uniform(0.0, np.log(9000.0)))),
                 res=bool(rng.integers(2)), wy=bool(rng.integers(2))) for i in range(n)]


@pytest.mark.parametrize("case", _draw_decode_cases(), ids=lambda c: "{i}-{M}x{H}x{N}".format(**c))
def test_random_decode_step_matches_the_two_calls(case):
    """The fused decode step over random row counts, hidden sizes and weight
    heights, to the bars of the fixed decode cases (the op's outputs bit for
    bit those of the separate op call; the linear within the GEMM bar of the
    oracle's exact product, bit for bit the two-call GEMM where both run the
    same reduction)."""
    from tests.test_gpu_decode import test_fused_decode_matches_the_two_calls as check
    c = case
    print(f"random decode case {c['i']}", flush=True)
    check(c["dt"], c["M"], c["H"], c["N"], c["res"], c["wy"])
