"""The C ABI's host-side argument checks (csrc/gnq_validate.hpp) built on
their own with g++'s address and undefined-behaviour sanitizers (any report
aborts the run), driven through overflow-prone corner cases and a seeded
fuzz of extreme sizes, enums and addresses.  Every status is compared with
the production library's for the calls it answers without a launch."""

import os
import random
import shutil
import subprocess

import pytest

from fp4_activation_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "validate_driver.cpp")
CSRC = os.path.join(ROOT, "fp4_activation_quant_amd", "csrc")

I64 = [0, 1, -1, 2, 7, 15, 16, 17, 31, 32, 48, 63, 64, 65, 96, 127, 128, 129, 255, 256, 4096, 5120,
       2**24, 2**24 + 32, 2**30, 2**30 + 64, 2**31 - 1, 2**31, 2**40, 2**59, 2**60, 2**60 + 1, 2**62,
       2**63 - 1, -2**63, -2**31]
ROW_BYTES = [0, 1, 4, 16, 64, 128, 1000, 4096, 2**20, 2**30, 2**40, 2**60, 2**63 - 1, -1, -2**63]
ADDRS = [0, 1, 2, 4, 8, 16, 0x1000, 0x10000000, 0x10000002, 0x10000800, 0x11000000, 0x12000000,
         0x13000000, 0x14000000, 0x15000000, 0x16000000, 2**47, 2**63, 2**64 - 16, 2**64 - 1]
PARAMS = ["0", "1", "7.5", "247", "248", "-1", "1e30", "nan", "inf"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "validate_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        if "asan" in r.stderr.lower() or "ubsan" in r.stderr.lower():
            pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
        raise AssertionError(r.stderr)
    return exe


def _run(exe, lines):
    """Statuses the sanitized checks print, one per line; any sanitizer
    report fails the test."""
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-2000:]
    out = r.stdout.split()
    assert len(out) == len(lines)
    return [int(v) for v in out]


def _u(v):
    """An address as the unsigned 64-bit value the C ABI receives."""
    return v % 2**64


def _line(cmd, a):
    if cmd == "fdec":
        x, r, ro, w, sc, M, H, dt, wy, q, y, b, bs, N, out = a
        return "fdec " + " ".join(str(v) for v in (_u(x), _u(r), _u(ro), _u(w), _u(sc), M, H, dt, wy, _u(q), _u(y),
                                                   _u(b), _u(bs), N, _u(out)))
    if cmd in ("op", "quant", "gemm", "gemm4"):
        return cmd + " " + " ".join(str(_u(v)) for v in a)
    if cmd == "traffic":
        nums = a[:6] + [_u(v) for v in a[6:8]] + a[8:10] + [_u(v) for v in a[10:14]] + a[14:18]
        return "traffic " + " ".join(str(v) for v in nums)
    if cmd == "probe":
        kind, inp, n, param, out = a
        return f"probe {kind} {_u(inp)} {n} {param} {_u(out)}"
    return f"bsb {a[0]} {a[1]}"


def _fuzz(n, seed):
    """(command, arguments) with signed sizes; addresses may be negative
    Python ints standing for their 64-bit patterns."""
    rng = random.Random(seed)
    pick = rng.choice
    out = []
    for _ in range(n):
        k = rng.randrange(8)
        if k == 0:       # x r w s M H dtype norm mode write_y q bs y
            out.append(("op", [pick(ADDRS) for _ in range(4)] +
                        [pick(I64), pick(I64), pick([-1, 0, 1, 2]), pick([-1, 0, 1, 2]),
                         pick([-1, 0, 1, 2, 3, 4]), pick([0, 1, 2])] + [pick(ADDRS) for _ in range(3)]))
        elif k == 1:     # y s M H dtype mode q bs
            out.append(("quant", [pick(ADDRS), pick(ADDRS), pick(I64), pick(I64), pick([-1, 0, 1, 2]),
                                  pick([0, 1, 3]), pick(ADDRS), pick(ADDRS)]))
        elif k == 2:     # mx a sa as b sb bs M N K out
            out.append(("gemm", [pick([0, 1])] + [pick(ADDRS) for _ in range(6)] +
                        [pick(I64), pick(I64), pick(I64), pick(ADDRS)]))
        elif k == 3:     # a sa ags b sb bgs M N K out
            out.append(("gemm4", [pick(ADDRS) for _ in range(6)] + [pick(I64), pick(I64), pick(I64), pick(ADDRS)]))
        elif k == 4:     # nsrc ndst rows threads grid flags src0 src1 srb0 srb1 dst0..3 drb0..3
            out.append(("traffic", [pick([-1, 0, 1, 2, 3]), pick([-1, 0, 1, 4, 5]), pick(I64 + [128, 256]),
                                    pick([0, 32, 64, 96, 256, 1024, 2048]), pick([-1, 0, 8, 2**31 - 1]),
                                    pick([-1, 0, 1, 2, 3, 4])] +
                        [pick(ADDRS), pick(ADDRS), pick(ROW_BYTES), pick(ROW_BYTES)] +
                        [pick(ADDRS) for _ in range(4)] + [pick(ROW_BYTES) for _ in range(4)]))
        elif k == 5:     # kind in n param out
            out.append(("probe", [pick([-1, 0, 5, 8, 9, 10]), pick(ADDRS), pick(I64), pick(PARAMS), pick(ADDRS)]))
        elif k == 6:     # M H
            out.append(("bsb", [pick(I64), pick(I64)]))
        else:            # x r ro w s M H dtype write_y q y b bs N out
            out.append(("fdec", [pick(ADDRS) for _ in range(5)] +
                        [pick(I64 + [1, 3, 8, 9]), pick(I64 + [1024, 2048, 4096]), pick([-1, 0, 1, 2]),
                         pick([0, 1])] + [pick(ADDRS) for _ in range(4)] + [pick(I64), pick(ADDRS)]))
    return out


def _library(cmd, a, st):
    """The production library's status for the same call when it returns
    without a launch (the checks reject it, or the problem is empty); None
    where it would launch a kernel."""
    L = _lib.lib()
    if cmd == "op":
        x, r, w, s, M, H, dt, norm, mode, wy, q, bs, y = a
        if st == _lib.NQ_OK and M != 0:
            return None
        return L.nq_add_rms_norm_quant(_u(x), _u(r), _u(w), 1e-6, _u(s), M, H, dt, norm, mode, wy, _u(q),
                                       _u(bs), _u(y), None)
    if cmd == "quant":
        y, s, M, H, dt, mode, q, bs = a
        if st == _lib.NQ_OK and M != 0:
            return None
        if mode == 0:
            return L.nq_quant_fp8_static(_u(y), _u(s), M, H, dt, _u(q), None)
        if mode == 1:
            return L.nq_quant_nvfp4(_u(y), _u(s), M, H, dt, _u(q), _u(bs), None)
        return L.nq_quant_mxfp8(_u(y), M, H, dt, _u(q), _u(bs), None)
    if cmd == "gemm":
        mx, A, sa, as_, B, sb, bs_, M, N, K, out = a
        if st == _lib.NQ_OK and M != 0 and N != 0:
            return None
        if mx:
            return L.nq_gemm_mxfp8(_u(A), _u(sa), _u(B), _u(sb), M, N, K, _u(out), None)
        # the static entry passes no block-scale buffers: compare only when they are null
        if sa or sb:
            return None
        return L.nq_gemm_fp8_static(_u(A), _u(as_), _u(B), _u(bs_), M, N, K, _u(out), None)
    if cmd == "gemm4":
        A, sa, ags, B, sb, bgs, M, N, K, out = a
        if st == _lib.NQ_OK and M != 0 and N != 0:
            return None
        return L.nq_gemm_nvfp4(_u(A), _u(sa), _u(ags), _u(B), _u(sb), _u(bgs), M, N, K, _u(out), None)
    if cmd == "traffic":
        nsrc, ndst, rows, threads, grid, flags = a[:6]
        if st == _lib.NQ_OK and rows != 0:
            return None
        if not (1 <= nsrc <= 2 and 0 <= ndst <= 4):
            return None          # the raw call takes the stream lists' own lengths
        src, srb = [_u(v) for v in a[6:6 + nsrc]], a[8:8 + nsrc]
        dst, drb = [_u(v) for v in a[10:10 + ndst]], a[14:14 + ndst]
        return _lib.nq_traffic_probe(src, srb, dst, drb, rows, threads, grid, flags, None)
    if cmd == "probe":
        kind, inp, n, param, out = a
        if st == _lib.NQ_OK and n != 0:
            return None
        return L.nq_convert_probe(kind, _u(inp), n, float(param), _u(out), None)
    if cmd == "fdec":
        x, r, ro, w, sc, M, H, dt, wy, q, y, b, bs, N, out = a
        if st == _lib.NQ_OK and M != 0:
            return None
        return L.nq_gemma_add_rms_norm_quant_gemm_fp8(_u(x), _u(r), _u(ro), _u(w), 1e-6, _u(sc), M, H, dt, wy,
                                                      _u(q), _u(y), _u(b), _u(bs), N, _u(out), None)
    return L.nq_block_scale_bytes(*a)


def test_sanitized_checks_match_the_library(driver):
    cases = _fuzz(30000, 11)
    got = _run(driver, [_line(c, a) for c, a in cases])
    compared = 0
    for (c, a), st in zip(cases, got):
        lib = _library(c, a, st)
        if lib is None:
            continue
        compared += 1
        assert lib == st, (c, a, lib, st)
    assert compared > 10000


def test_sanitized_corner_cases(driver):
    """Fixed expectations where 64-bit sizes could overflow."""
    X, R, W, S, Q, B, Y = (0x10000000 + i * 0x1000000 for i in range(7))
    lines = [
        "bsb 9223372036854775807 64",                     # M near 2^63: a size the entry points reject
        "bsb 1 16",
        "bsb 129 5120",
        f"op {X} {R} {W} {S} 4 128 0 0 0 0 {Q} {B} {Y}",
        f"op {X} {2**64 - 16} {W} {S} 1 128 0 0 0 0 {Q} {B} {Y}",     # residual past the address space
        f"op {X} {R} {W} {S} {2**63 - 1} {2**30} 0 0 1 1 {Q} {B} {Y}",
        f"quant {X} {S} {2**63 - 1} 64 0 1 {Q} {B}",
        f"gemm 1 {X} {R} {W} {S} {Q} {B} {2**30} {2**30} {2**24} {Y}",
        f"gemm4 {X} {R} {W} {S} {Q} {B} {2**30} {2**30} {2**24} {Y}",
        f"probe 8 {X} 16 1e30 {Y}",
        f"probe 8 {X} 16 nan {Y}",
    ]
    got = _run(driver, lines)
    assert got[0] == 0 and got[1] == 128 * 4 and got[2] == 256 * 320
    assert got[3] == _lib.NQ_OK
    assert got[4:] == [_lib.NQ_EINVAL] * 7
    assert _lib.nq_block_scale_bytes(2**63 - 1, 64) == 0
