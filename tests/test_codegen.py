"""Checks on the gfx950 code the compiler emits for the fused kernels (CPU
only: hipcc cross-compiles to AMD assembly here, nothing runs).

y = RN_D(fl32(t * g)) rounds the fp32 product, then rounds that to the
activation dtype.  A fused multiply-round instruction (v_fma_mixlo_f16 and
its relatives) rounds the exact product once instead, and with the +0 addend
the compiler gives it turns a -0 product into +0.  The compiler forms it from
a product feeding a lone fp16 conversion, so no kernel may contain one.
"""

import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from fp4_activation_quant_amd import build as B

FUSED_MULTIPLY_ROUND = re.compile(r"\bv_(fma|mad)_mix(lo|hi)_(f16|bf16)\b")
UNITS = ["gnq_fused_fp16_fp8.hip", "gnq_fused_fp16_nvfp4.hip", "gnq_fused_fp16_mxfp8.hip",
         "gnq_fused_fp16_none.hip", "gnq_fused_bf16_fp8.hip", "gnq_quant.hip", "gnq_decode.hip"]


def _assembly(unit, tmp):
    out = os.path.join(tmp, unit + ".s")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC,
           "--cuda-device-only", "-S", os.path.join(B.CSRC, unit), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    with open(out) as f:
        return f.read()


def test_no_fused_multiply_round_in_the_kernels():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory(prefix="gnq_asm_") as tmp:
        with cf.ThreadPoolExecutor(min(len(UNITS), os.cpu_count() or 4)) as ex:
            asm = dict(zip(UNITS, ex.map(lambda u: _assembly(u, tmp), UNITS)))
    found = {u: sorted(set(m.group(0) for m in FUSED_MULTIPLY_ROUND.finditer(a))) for u, a in asm.items()}
    assert not any(found.values()), found
