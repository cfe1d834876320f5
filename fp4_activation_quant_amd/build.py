"""Build the gfx950 HIP library in-tree: fp4_activation_quant_amd/libgemma_norm_quant.so.

    python -m fp4_activation_quant_amd.build

Each csrc/*.hip translation unit (one per activation dtype and output mode
for the fused kernels, one for the standalone quant, one for the C ABI) is
compiled in parallel, then linked into one shared library.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgemma_norm_quant.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE fp32 everywhere: no contraction, correctly rounded divide/sqrt,
    # denormals kept (the defaults, stated explicitly).
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # No packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=True, jobs=None) -> str:
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="gnq_build_") as tmp:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([cc, *HIPCC_FLAGS, *inc, "-c", src, "-o", obj])
        jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
        if verbose:
            print(f"compiling {len(cmds)} translation units ({jobs} parallel)", flush=True)
        with cf.ThreadPoolExecutor(jobs) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = LIB + ".tmp"
        # -z defs: an unresolved symbol (e.g. a kernel template never
        # instantiated) fails the link instead of the first call.
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
