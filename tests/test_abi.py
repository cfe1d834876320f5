"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and its host-side logic (sizes, status strings, argument
validation, the M == 0 early return) behaves as documented.  No call here
reaches a kernel launch."""

import ctypes
import os
import re

import pytest

from fp4_activation_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma_norm_quant.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", src)))


def test_library_is_built():
    assert os.path.exists(_lib.LIB_PATH), "run python -m fp4_activation_quant_amd.build"


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    L = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert _lib.nq_abi_version() == 7
    assert _lib.nq_status_string(0) == "ok"
    for s in range(0, 6):
        assert isinstance(_lib.nq_status_string(s), str)


@pytest.mark.parametrize("M,H,want", [(1, 64, 512), (128, 64, 512), (129, 64, 1024),
                                      (8192, 4096, 8192 * 256), (4096, 5120, 4096 * 320),
                                      (32768, 8192, 32768 * 512), (1, 80, 128 * 8),
                                      (0, 64, 0), (5, 8, 0)])
def test_block_scale_bytes(M, H, want):
    assert _lib.nq_block_scale_bytes(M, H) == want


# Fake, never-dereferenced device addresses: every case below must be
# rejected (or return early) on the host.
X, R, W, S, Q, B, Y = (0x10000000 + i * 0x1000000 for i in range(7))


def call(**over):
    a = dict(x=X, r=R, w=W, eps=1e-6, s=S, M=4, H=128, dtype=0, mode=0, wy=0, q=Q, bs=B, y=Y)
    a.update(over)
    return _lib.nq_gemma_add_rms_norm_quant(a["x"], a["r"], a["w"], a["eps"], a["s"], a["M"],
                                            a["H"], a["dtype"], a["mode"], a["wy"], a["q"],
                                            a["bs"], a["y"], 0)


@pytest.mark.parametrize("over,want", [
    (dict(x=0), _lib.NQ_EINVAL),
    (dict(w=0), _lib.NQ_EINVAL),
    (dict(s=0), _lib.NQ_EINVAL),
    (dict(q=0), _lib.NQ_EINVAL),
    (dict(M=-3), _lib.NQ_EINVAL),
    (dict(H=0), _lib.NQ_EINVAL),
    (dict(H=-5), _lib.NQ_EINVAL),
    (dict(H=(1 << 30) + 64), _lib.NQ_EINVAL),          # H beyond 2^30
    (dict(M=(1 << 60) // 128 + 1), _lib.NQ_EINVAL),    # M * H beyond 2^60 (H = 128)
    (dict(dtype=7), _lib.NQ_EINVAL),
    (dict(mode=-1), _lib.NQ_EINVAL),
    (dict(wy=1, y=0), _lib.NQ_EINVAL),
    (dict(mode=1, bs=0), _lib.NQ_EINVAL),
    (dict(mode=1, H=96), _lib.NQ_EUNSUPPORTED),
    (dict(mode=1, H=32), _lib.NQ_EUNSUPPORTED),
    (dict(r=X), _lib.NQ_EINVAL),
    (dict(r=X + 256), _lib.NQ_EINVAL),
    (dict(q=X + 100), _lib.NQ_EINVAL),
    (dict(wy=1, y=R + 2), _lib.NQ_EINVAL),
    (dict(mode=1, bs=Q + 10), _lib.NQ_EINVAL),
    (dict(x=X + 1), _lib.NQ_EINVAL),                 # 16-bit data must be 2-byte aligned
    (dict(w=W + 1), _lib.NQ_EINVAL),
    (dict(wy=1, y=Y + 3), _lib.NQ_EINVAL),
    (dict(s=S + 2), _lib.NQ_EINVAL),                 # fp32 scale must be 4-byte aligned
    # outputs overlapping the weight (H * 2 bytes) or the fp32 scale
    (dict(q=W + 64), _lib.NQ_EINVAL),
    (dict(r=W - 1024 + 2), _lib.NQ_EINVAL),          # residual's last bytes reach the weight
    (dict(wy=1, y=W + 254), _lib.NQ_EINVAL),
    (dict(mode=1, bs=W + 16), _lib.NQ_EINVAL),
    (dict(q=S - 508), _lib.NQ_EINVAL),               # codes (512 bytes) end inside the scale
    (dict(mode=1, bs=S), _lib.NQ_EINVAL),
    (dict(r=S + 0), _lib.NQ_EINVAL),
    (dict(wy=1, y=S - 1022), _lib.NQ_EINVAL),
    # M == 0: valid, returns before any launch
    (dict(M=0), _lib.NQ_OK),
    (dict(M=0, mode=1, wy=1), _lib.NQ_OK),
    (dict(M=0, r=0), _lib.NQ_OK),
])
def test_validation(over, want):
    assert call(**over) == want


def call_ex(**over):
    a = dict(x=X, r=R, w=W, eps=1e-6, s=S, M=4, H=128, dtype=0, norm=0, mode=0, wy=0, q=Q, bs=B, y=Y)
    a.update(over)
    return _lib.nq_add_rms_norm_quant(a["x"], a["r"], a["w"], a["eps"], a["s"], a["M"], a["H"],
                                      a["dtype"], a["norm"], a["mode"], a["wy"], a["q"], a["bs"],
                                      a["y"], 0)


@pytest.mark.parametrize("over,want", [
    (dict(norm=2), _lib.NQ_EINVAL),
    (dict(mode=4), _lib.NQ_EINVAL),
    (dict(mode=3, bs=0), _lib.NQ_EINVAL),             # MXFP8 needs its scale buffer
    (dict(mode=3, q=0), _lib.NQ_EINVAL),
    (dict(mode=3, H=48), _lib.NQ_EUNSUPPORTED),       # H % 32 != 0
    (dict(mode=3, H=16, M=0), _lib.NQ_EUNSUPPORTED),
    (dict(mode=3, bs=Q + 500), _lib.NQ_EINVAL),       # scales overlap the (M, H) codes
    (dict(mode=3, bs=R + 8), _lib.NQ_EINVAL),         # scales overlap residual
    (dict(mode=3, wy=1, y=B + 8), _lib.NQ_EINVAL),    # y overlaps the scales
    (dict(mode=3, s=0, M=0), _lib.NQ_OK),             # scale ignored for MXFP8
    (dict(mode=3, H=96, M=0, norm=1), _lib.NQ_OK),
    (dict(mode=2, wy=0), _lib.NQ_EINVAL),            # no-quant mode needs y
    (dict(mode=2, wy=1, y=0), _lib.NQ_EINVAL),
    (dict(mode=2, wy=1, y=X + 64), _lib.NQ_EINVAL),  # y overlaps x
    (dict(mode=2, wy=1, s=0, q=0, bs=0, M=0), _lib.NQ_OK),   # scale/q ignored in no-quant mode
    (dict(mode=3, bs=W + 2), _lib.NQ_EINVAL),         # MXFP8 scales overlap the weight
    (dict(mode=2, wy=1, y=W - 1000), _lib.NQ_EINVAL),  # y overlaps the weight
    (dict(norm=1, mode=1, H=96), _lib.NQ_EUNSUPPORTED),
    (dict(norm=1, M=0), _lib.NQ_OK),
    (dict(x=0, norm=1), _lib.NQ_EINVAL),
])
def test_general_entry_validation(over, want):
    assert call_ex(**over) == want


def test_gemma_entry_rejects_no_quant_and_mxfp8_modes():
    assert call(mode=2, wy=1, M=0) == _lib.NQ_EINVAL
    assert call(mode=3, M=0) == _lib.NQ_EINVAL


@pytest.mark.parametrize("nv,over,want", [
    (False, dict(y=0), _lib.NQ_EINVAL),
    (False, dict(s=0), _lib.NQ_EINVAL),
    (False, dict(q=0), _lib.NQ_EINVAL),
    (False, dict(dtype=5), _lib.NQ_EINVAL),
    (False, dict(H=0), _lib.NQ_EINVAL),
    (False, dict(q=X + 10), _lib.NQ_EINVAL),          # q overlaps y
    (False, dict(M=0), _lib.NQ_OK),
    (False, dict(H=7, M=0), _lib.NQ_OK),             # any H for FP8
    (False, dict(M=1 << 59), _lib.NQ_EINVAL),        # M * H beyond 2^60
    (True, dict(bs=0), _lib.NQ_EINVAL),
    (True, dict(H=24), _lib.NQ_EUNSUPPORTED),
    (True, dict(H=48, M=0), _lib.NQ_OK),             # H % 16 == 0 suffices standalone
    (True, dict(bs=Q + 4), _lib.NQ_EINVAL),
    (False, dict(s=Q + 4), _lib.NQ_EINVAL),           # scale inside the codes
    (True, dict(s=B + 8), _lib.NQ_EINVAL),            # global scale inside the scale buffer
    (True, dict(s=Q + 252), _lib.NQ_EINVAL),          # global scale inside the codes
])
def test_standalone_quant_validation(nv, over, want):
    a = dict(y=X, s=S, M=4, H=128, dtype=0, q=Q, bs=B)
    a.update(over)
    if nv:
        st = _lib.nq_quant_nvfp4(a["y"], a["s"], a["M"], a["H"], a["dtype"], a["q"], a["bs"], 0)
    else:
        st = _lib.nq_quant_fp8_static(a["y"], a["s"], a["M"], a["H"], a["dtype"], a["q"], 0)
    assert st == want


@pytest.mark.parametrize("over,want", [
    (dict(y=0), _lib.NQ_EINVAL),
    (dict(q=0), _lib.NQ_EINVAL),
    (dict(bs=0), _lib.NQ_EINVAL),
    (dict(H=48), _lib.NQ_EUNSUPPORTED),
    (dict(dtype=2), _lib.NQ_EINVAL),
    (dict(bs=Q + 511), _lib.NQ_EINVAL),               # scales overlap the codes
    (dict(q=X + 2), _lib.NQ_EINVAL),                  # codes overlap y
    (dict(M=0), _lib.NQ_OK),
    (dict(M=0, H=32), _lib.NQ_OK),
])
def test_standalone_mxfp8_validation(over, want):
    a = dict(y=X, M=4, H=128, dtype=0, q=Q, bs=B)
    a.update(over)
    assert _lib.nq_quant_mxfp8(a["y"], a["M"], a["H"], a["dtype"], a["q"], a["bs"], 0) == want


def test_probe_validation():
    assert _lib.nq_convert_probe(12, 0x1000, 4, 1.0, 0x2000, 0) == _lib.NQ_EINVAL
    for kind in (10, 11):
        assert _lib.nq_convert_probe(kind, 0x1000, 12, 1.0, 0x2000, 0) == _lib.NQ_EINVAL
        assert _lib.nq_convert_probe(kind, 0x1000, 0, 1.0, 0x2000, 0) == _lib.NQ_OK
    assert _lib.nq_convert_probe(-1, 0x1000, 4, 1.0, 0x2000, 0) == _lib.NQ_EINVAL
    for bad in (-1.0, 248.0, 12.5, float("nan"), float("inf")):
        assert _lib.nq_convert_probe(8, 0x1000, 4, bad, 0x2000, 0) == _lib.NQ_EINVAL, bad
    assert _lib.nq_convert_probe(8, 0x1000, 0, 247.0, 0x2000, 0) == _lib.NQ_OK
    assert _lib.nq_convert_probe(0, 0x1000, -1, 1.0, 0x2000, 0) == _lib.NQ_EINVAL
    assert _lib.nq_convert_probe(0, 0, 4, 1.0, 0x2000, 0) == _lib.NQ_EINVAL
    assert _lib.nq_convert_probe(0, 0x1000, 0, 1.0, 0x2000, 0) == _lib.NQ_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_torch_wrapper_rejects_bad_tensors_before_the_library():
    """The torch-facing wrapper checks its arguments itself (ValueError) and
    never reaches the library with host tensors or mismatched shapes."""
    import torch
    from fp4_activation_quant_amd import ops
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    w = torch.zeros(128, dtype=torch.bfloat16)
    s = torch.ones(1, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        ops.gemma_add_rms_norm_quant(x, None, w, 1e-6, s, False)
    with pytest.raises(ValueError, match="device"):
        ops.add_rms_norm_quant(x, None, w, 1e-6, None, "mxfp8")
    with pytest.raises(ValueError):
        ops.quant_mxfp8(x)


@pytest.mark.parametrize("mx", [True, False])
@pytest.mark.parametrize("over,want", [
    (dict(a=0), _lib.NQ_EINVAL),
    (dict(b=0), _lib.NQ_EINVAL),
    (dict(out=0), _lib.NQ_EINVAL),
    (dict(sa=0), _lib.NQ_EINVAL),
    (dict(sb=0), _lib.NQ_EINVAL),
    (dict(K=0), _lib.NQ_EINVAL),
    (dict(M=-1), _lib.NQ_EINVAL),
    (dict(K=48), _lib.NQ_EUNSUPPORTED),
    (dict(a=X + 8), _lib.NQ_EINVAL),                  # unaligned codes
    (dict(out=X + 64), _lib.NQ_EINVAL),               # out overlaps a
    (dict(out=Q + 4096), _lib.NQ_EINVAL),             # out overlaps b
    (dict(out=Y + 1), _lib.NQ_EINVAL),                # bf16 output must be 2-byte aligned
    (dict(M=1 << 30, N=1 << 30, out=0x7F0000000000), _lib.NQ_EINVAL),  # tile count beyond a grid
    (dict(M=0), _lib.NQ_OK),
    (dict(N=0), _lib.NQ_OK),
])
def test_gemm_validation(mx, over, want):
    a = dict(a=X, sa=S, b=Q, sb=B, M=4, N=8, K=4096, out=Y)
    a.update(over)
    fn = _lib.nq_gemm_mxfp8 if mx else _lib.nq_gemm_fp8_static
    assert fn(a["a"], a["sa"], a["b"], a["sb"], a["M"], a["N"], a["K"], a["out"], 0) == want


@pytest.mark.parametrize("over,want", [
    (dict(a=0), _lib.NQ_EINVAL),
    (dict(b=0), _lib.NQ_EINVAL),
    (dict(sa=0), _lib.NQ_EINVAL),
    (dict(sb=0), _lib.NQ_EINVAL),
    (dict(ga=0), _lib.NQ_EINVAL),
    (dict(gb=0), _lib.NQ_EINVAL),
    (dict(out=0), _lib.NQ_EINVAL),
    (dict(K=0), _lib.NQ_EINVAL),
    (dict(N=-1), _lib.NQ_EINVAL),
    (dict(K=96), _lib.NQ_EUNSUPPORTED),                # K % 64 != 0
    (dict(sa=S + 8), _lib.NQ_EINVAL),                 # scale buffer not 16-byte aligned
    (dict(ga=S + 2), _lib.NQ_EINVAL),                 # global scale not 4-byte aligned
    (dict(out=X + 64), _lib.NQ_EINVAL),               # out overlaps a
    (dict(out=Y + 1), _lib.NQ_EINVAL),
    (dict(M=1 << 30, N=1 << 30, out=0x7F0000000000), _lib.NQ_EINVAL),  # tile count beyond a grid
    (dict(M=0), _lib.NQ_OK),
    (dict(N=0), _lib.NQ_OK),
])
def test_gemm_nvfp4_validation(over, want):
    a = dict(a=X, sa=S, ga=B, b=Q, sb=B + 4096, gb=B + 64, M=4, N=8, K=4096, out=Y)
    a.update(over)
    assert _lib.nq_gemm_nvfp4(a["a"], a["sa"], a["ga"], a["b"], a["sb"], a["gb"], a["M"], a["N"], a["K"],
                              a["out"], 0) == want


SA, SB, DA, DB = (0x30000000 + i * 0x1000000 for i in range(4))


@pytest.mark.parametrize("over,want", [
    (dict(), None),                                         # valid: only M = 0 returns before a launch
    (dict(src=[]), _lib.NQ_EINVAL),                         # 1 or 2 read streams
    (dict(src=[SA, SB, SA + 0x100000], srb=[1024] * 3), _lib.NQ_EINVAL),
    (dict(dst=[DA] * 5, drb=[64] * 5), _lib.NQ_EINVAL),     # at most 4 write streams
    (dict(srb=[1000]), _lib.NQ_EINVAL),                     # row bytes a multiple of 16
    (dict(drb=[0]), _lib.NQ_EINVAL),
    (dict(srb=[64 * 256 + 16]), _lib.NQ_EINVAL),            # a read row beyond 4 chunks per thread
    (dict(threads=96), _lib.NQ_EINVAL),
    (dict(threads=2048), _lib.NQ_EINVAL),
    (dict(grid=-1), _lib.NQ_EINVAL),
    (dict(src=[SA + 8]), _lib.NQ_EINVAL),                   # 16-byte alignment
    (dict(dst=[0]), _lib.NQ_EINVAL),
    (dict(dst=[SA + 512], rows=8), _lib.NQ_EINVAL),         # a write stream over a read stream
    (dict(dst=[DA, DA + 256], drb=[64, 64], rows=8), _lib.NQ_EINVAL),   # write streams overlapping
    (dict(rows=-1), _lib.NQ_EINVAL),
    (dict(pf=4), _lib.NQ_EINVAL),                           # unknown flag bit
    (dict(pf=-1), _lib.NQ_EINVAL),
    (dict(pf=3), None),                                     # prefetch + tiled scales (M = 0: no launch)
    (dict(pf=2, rows=130), _lib.NQ_EINVAL),                 # tiled scales on whole 128-row tiles only
    (dict(pf=2, dst=[], drb=[], rows=128), _lib.NQ_EINVAL), # and a write stream to hold them
])
def test_traffic_probe_validation(over, want):
    a = dict(src=[SA], srb=[1024], dst=[DA], drb=[512], rows=0, threads=256, grid=0, pf=0)
    a.update(over)
    if want is None:
        want = _lib.NQ_OK
    assert _lib.nq_traffic_probe(a["src"], a["srb"], a["dst"], a["drb"], a["rows"], a["threads"],
                                 a["grid"], a["pf"], 0) == want


def test_traffic_probe_nonzero_rows_still_validated():
    # rows > 0 with a bad stream is rejected before any launch
    assert _lib.nq_traffic_probe([SA], [1000], [DA], [512], 8, 256, 0, 0, 0) == _lib.NQ_EINVAL
    assert _lib.nq_traffic_probe([SA], [1024], [SA], [512], 8, 256, 0, 0, 0) == _lib.NQ_EINVAL


FX, FR, FRO, FW, FS, FQ, FY, FB, FBS, FO = (0x40000000 + i * 0x1000000 for i in range(10))


@pytest.mark.parametrize("over,want", [
    (dict(M=0), _lib.NQ_OK),                          # nothing to do
    (dict(M=9), _lib.NQ_EUNSUPPORTED),                # more than 8 rows
    (dict(H=5120), _lib.NQ_EUNSUPPORTED),
    (dict(N=0), _lib.NQ_EUNSUPPORTED),
    (dict(M=-1), _lib.NQ_EINVAL),
    (dict(dtype=3), _lib.NQ_EINVAL),
    (dict(x=0), _lib.NQ_EINVAL),
    (dict(b=0), _lib.NQ_EINVAL),
    (dict(ro=0), _lib.NQ_EINVAL),                     # residual without residual_out
    (dict(r=0), _lib.NQ_EINVAL),                      # residual_out without residual
    (dict(ro=FR), _lib.NQ_EINVAL),                    # in place
    (dict(wy=1, y=0), _lib.NQ_EINVAL),
    (dict(x=FX + 8), _lib.NQ_EINVAL),                 # 16-byte alignment
    (dict(q=FQ + 4), _lib.NQ_EINVAL),
    (dict(o=FB + 100), _lib.NQ_EINVAL),               # out over the weight
    (dict(q=FW), _lib.NQ_EINVAL),                     # q over the norm weight
    (dict(o=FS - 8), _lib.NQ_EINVAL),                 # out over the scale
])
def test_fused_decode_validation(over, want):
    a = dict(x=FX, r=FR, ro=FRO, w=FW, s=FS, M=4, H=4096, dtype=0, wy=0, q=FQ, y=FY, b=FB, bs=FBS, N=4096, o=FO)
    a.update(over)
    st = _lib.nq_gemma_add_rms_norm_quant_gemm_fp8(a["x"], a["r"], a["ro"], a["w"], 1e-6, a["s"], a["M"], a["H"],
                                                   a["dtype"], a["wy"], a["q"], a["y"], a["b"], a["bs"], a["N"],
                                                   a["o"], 0)
    assert st == want
