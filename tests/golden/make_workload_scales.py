"""Write tests/golden/workload_scales.json: each workload's fp32 quant scale.

Calls only the CPU oracle (plus the seeded input generator).  amax is
max |y| of the oracle's normed activation over the workload's draw (for the
decode sweep, over its separate calibration draw).  Static FP8 uses
s = fl32(amax / 448); NVFP4 uses the global scale gs = fl32(448 * 6 / amax).

    python tests/golden/make_workload_scales.py [name ...]
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
from fp4_activation_quant_amd.workloads import WORKLOADS, SCALES_JSON, make_inputs, make_calibration_inputs  # noqa: E402

FMT = {"bf16": O.BF16, "fp16": O.FP16}


def _bits(t):
    return t.contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def amax_of_y(x, r, w, eps, fmt, chunk=512):
    wb = _bits(w)
    amax = 0.0
    for i in range(0, x.shape[0], chunk):
        xb = _bits(x[i:i + chunk])
        h = O.add_residual(xb, _bits(r[i:i + chunk]), fmt) if r is not None else xb
        y = O.bits_to_f64(O.gemma_rms_norm(h, wb, eps, fmt), fmt)
        amax = max(amax, float(np.max(np.abs(y))))
    return amax


def main(names):
    table = {}
    if os.path.exists(SCALES_JSON):
        with open(SCALES_JSON) as f:
            table = json.load(f)
    for name in names:
        wl = WORKLOADS[name]
        if wl.scale_rule in ("fixed", "none"):
            continue
        if wl.scale_rule == "fp8_amax_calibration":
            x, r, w = make_calibration_inputs(wl)
        else:
            x, r, w = make_inputs(wl)
        amax = amax_of_y(x, r, w, wl.eps, FMT[wl.dtype])
        if wl.scale_rule.startswith("fp8"):
            s = np.float32(np.float32(amax) / np.float32(448.0))
        else:
            s = np.float32(448.0 * 6.0 / amax)
        table[name] = {"amax": amax, "scale": float(s), "scale_hex": float(s).hex(),
                       "rule": wl.scale_rule}
        print(name, amax, float(s), flush=True)
    with open(SCALES_JSON, "w") as f:
        json.dump(dict(sorted(table.items())), f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))
