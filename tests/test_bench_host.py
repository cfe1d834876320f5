"""Host logic of bench.py without a GPU: the algorithmic byte count that the
roofline's `achieved` divides by, and the refusal of a multi-GPU run."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from fp4_activation_quant_amd.workloads import WORKLOADS  # noqa: E402

# Bytes per call, worked out by hand from the op's traffic: read x (2 bytes
# per element) and the residual (2), write the residual back (2), y (2) when
# it is written, and the codes (FP8: 1 byte per element; NVFP4: 1/2 plus one
# scale byte per 16 elements); once per call the weight (2 H) and the
# 4-byte scale.  E.g. M = 16, H = 2048, FP8 with residual and y:
# 16 * 2048 * 9 + 2 * 2048 + 4 = 299012.
EXPECTED = {
    "fp8_m16_h2048_bf16_y": 299_012,
    "fp8_decode_m1_h4096_bf16": 36_868,
    "fp8_decode_m8_h4096_bf16": 237_572,
    "fp8_decode_m64_h4096_bf16": 1_843_204,
    "fp8_decode_m256_h4096_bf16": 7_348_228,
    "nvfp4_prefill_m8192_h4096_bf16_y": 287_318_020,
    "fp8_res_m4096_h5120_fp16": 146_810_884,
    "fp8_nores_m4096_h5120_fp16": 62_924_804,
    "nvfp4_res_m4096_h5120_fp16": 137_635_844,
    "nvfp4_nores_m4096_h5120_fp16": 53_749_764,
    "nvfp4_m32768_h8192_bf16_y": 2_298_494_980,
}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    rd, wr = bench.algorithmic_bytes(WORKLOADS[name])
    assert rd + wr == EXPECTED[name]


def test_mxfp8_bytes_have_no_scale_read_and_one_code_byte_per_element():
    wl = WORKLOADS["mxfp8_m32768_h8192_bf16_y"]
    rd, wr = bench.algorithmic_bytes(wl)
    MH = wl.M * wl.H
    assert rd == 4 * MH + 2 * wl.H                       # x, residual, weight; no scale
    assert wr == 2 * MH + 2 * MH + MH + MH // 32         # residual, y, codes, E8M0 scales


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("H,cpt", [(16, 1), (2048, 1), (4096, 1), (5120, 2), (6144, 1), (8192, 1),
                                   (8320, 2), (16384, 2), (16512, 4), (32768, 4)])
def test_kernel_name_follows_the_launchers_chunk_rule(H, cpt):
    """One 8-element chunk per thread up to H = 4096 and wherever that makes
    a workgroup of whole 4-wave groups within 1024 threads; else two up to
    H = 16384, four beyond (the fused launcher's chunks_per_thread)."""
    assert bench.chunks_per_thread(H) == cpt
    assert bench.kernel_name(WORKLOADS["nvfp4_m32768_h8192_bf16_y"]).endswith(",1>")
    assert bench.kernel_name(WORKLOADS["fp8_nores_m4096_h5120_fp16"]).endswith(",2,prefetch>")
    assert bench.kernel_name(WORKLOADS["fp8_decode_m256_h4096_bf16"]).endswith(",1>")


@pytest.mark.parametrize("M,H,pf", [(4096, 5120, True), (2048, 4160, True), (16384, 6080, True),
                                    (2047, 5120, False), (16385, 5120, False), (4096, 4096, False),
                                    (4096, 6144, False), (32768, 8192, False), (1, 5120, False)])
def test_prefetch_rule(M, H, pf):
    """Rows of 4096 < H < 6144 at 2048 <= M <= 16384 take the looping
    prefetch launch (the fused launcher's prefetch_rows): two chunks per
    thread without a residual, and with one up to H = 5120."""
    assert bench.prefetch_rows(M, H) == pf
    if pf:
        assert bench.chunks_per_thread(H) == 2
        assert bench.chunks_per_thread(H, res=True) == (1 if H <= 5120 else 2)


@pytest.mark.parametrize("H,cpt", [(4096, 1), (4160, 1), (5120, 1), (5184, 2), (6144, 1), (8192, 1), (16384, 2)])
def test_residual_rows_chunk_rule(H, cpt):
    """Rows with a residual at 4096 < H <= 5120 take one chunk per thread in
    every launch form."""
    assert bench.chunks_per_thread(H, res=True) == cpt
    assert bench.kernel_name(WORKLOADS["fp8_res_m4096_h5120_fp16"]).endswith(",1,prefetch>")
    assert bench.kernel_name(WORKLOADS["nvfp4_nores_m4096_h5120_fp16"]).endswith(",2,prefetch>")
    assert bench.block_threads(5120, res=True) == 640 and bench.block_threads(5120) == 320


@pytest.mark.parametrize("M,N,K,kernel", [
    (1, 4096, 4096, "gemm_nvfp4_gemv"), (3, 4096, 4096, "gemm_nvfp4_gemv"),
    (4, 4096, 4096, "gemm_nvfp4_k<8,32,32,4>"), (2, 8192, 4096, "gemm_nvfp4_k<8,32,32,4>"),
    (8, 300, 2880, "gemm_nvfp4_gemv"), (8, 50, 8192, "gemm_nvfp4_k<8,32,32,4>"),
    (64, 4096, 4096, "gemm_nvfp4_k<8,32,32,4>"), (128, 4096, 4096, "gemm_nvfp4_k<8,64,32,4>"),
    (256, 4096, 4096, "gemm_nvfp4_k<8,64,64,3>"), (1024, 4096, 4096, "gemm_nvfp4_k<4,128,64,4>"),
    (2048, 4096, 4096, "gemm_nvfp4_big"), (8192, 4096, 4096, "gemm_nvfp4_big"),
    (300, 200, 448, "gemm_nvfp4_k<4,32,32,8>")])
def test_nvfp4_kernel_follows_the_dispatch(M, N, K, kernel):
    """The bench names the NVFP4 consumer kernel the library's tile choice
    picks (largest tile with enough workgroups)."""
    assert bench.nvfp4_kernel(M, N, K) == kernel


@pytest.mark.parametrize("M,N,K,kernel", [
    (1, 4096, 4096, "gemm_fp8_decode"), (256, 4096, 4096, "gemm_fp8_decode"),
    (192, 8192, 4096, "gemm_fp8_tn_dma<128>"), (300, 4096, 4096, "gemm_fp8_tn_dma<128>"),
    (1024, 4096, 4096, "gemm_fp8_tn_dma<128>"), (2048, 4096, 4096, "gemm_fp8_tn_dma<256>"),
    (8192, 4096, 4096, "gemm_fp8_tn_dma<256>"), (300, 520, 1056, "gemm_fp8_tn"),
    (33, 300, 1536, "gemm_fp8_skinny")])
def test_fp8_kernel_follows_the_dispatch(M, N, K, kernel):
    """The bench names the FP8 / MXFP8 consumer kernel the library's tile
    choice picks (256 x 256 once 128 workgroups, else 128 x 128 past 256 rows
    or at 128 workgroups, else the decode-size kernels)."""
    assert bench.fp8_kernel(M, N, K) == kernel


def test_cpu_baseline_single_and_all_threads(monkeypatch):
    """Both CPU-baseline legs run the oracle on a prefix of the rows: the
    single-threaded one and the one over every host thread (OMP_NUM_THREADS
    caps the count)."""
    from fp4_activation_quant_amd.workloads import make_inputs, load_scale
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert bench.host_threads() <= 2
    wl = WORKLOADS["fp8_m16_h2048_bf16_y"]
    x, r, w = make_inputs(wl)
    out = bench.cpu_baseline(wl, x, r, w, load_scale(wl), 0.05)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["value"] > 0
    if bench.host_threads() > 1:
        par = out["all_threads"]
        assert par["cores"] == 2 and par["value"] > 0 and par["unit"] == "GB/s"


def test_kernel_hash_ignores_comments_only():
    """Traffic counters stay attached to the fused kernel's code across
    comment and layout edits, and not across code edits."""
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow check */\n}\n"
    assert bench._code_only(a) == bench._code_only("int f(int x) {\n\n return 2 * x;\n}")
    assert bench._code_only(a) != bench._code_only("int f(int x) { return 3 * x; }")
    assert len(bench.kernel_sha()) == 16
