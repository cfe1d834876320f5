"""GPU parity over a seeded random sweep of the op's argument space, through
the C ABI: output mode (static FP8, NVFP4, MXFP8, none), activation dtype,
residual or not, write_y or not, Gemma or plain norm, misaligned views, and
shapes drawn across every launch form (several rows per wave for H <= 512,
one workgroup per row, the looping launch at 4096 < H < 6144 with 2048 <=
M <= 16384, the element-wise path for H % 16 != 0 or unaligned pointers).
Every case is compared with the oracle on every row, to the same bars as the
fixed workloads (tests/parity.py)."""

import numpy as np
import pytest
import torch

from fp4_activation_quant_amd import _lib
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
        cases.append(dict(i=i, mode=mode, dt=dt, res=res, wy=wy, norm=norm, M=M, H=H, misalign=misalign,
                          xs=xs, rs=rs, ws=ws, scale=scale, seed=SEED + 7919 * i))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "{i}-{mode}-{M}x{H}".format(**c))
def test_random_case_matches_oracle(case):
    c = case
    print(f"random case {c['i']}: {c['mode']} {c['dt']} M={c['M']} H={c['H']} res={c['res']} "
          f"write_y={c['wy']} norm={c['norm']} misalign={c['misalign']} scale={c['scale']:.6g}", flush=True)
    g = torch.Generator().manual_seed(c["seed"])
    M, H, dt = c["M"], c["H"], c["dt"]
    x = (torch.randn(M, H, generator=g) * c["xs"]).to(dt)
    r = (torch.randn(M, H, generator=g) * c["rs"]).to(dt) if c["res"] else None
    w = (torch.randn(H, generator=g) * c["ws"]).to(dt)
    mode = c["mode"]
    gpu = P.run_gpu(x, r.clone() if r is not None else None, w, 1e-6, c["scale"], mode == "nvfp4", c["wy"],
                    misalign=c["misalign"], norm=c["norm"], quant=mode != "none", mxfp8=mode == "mxfp8")
    rep = P.check(P.compare(gpu, x, r, w, 1e-6, c["scale"], P.all_rows(M)))
    print(rep, flush=True)
