"""GPU-vs-oracle comparison shared by the GPU tests and the smoke check.

The HIP op runs on device copies of CPU inputs, into output buffers that are
pre-filled with a sentinel byte and followed by guard bytes, so that writes
outside an output (or into the unwritten padding rows of the NVFP4 scale
buffer) show up.  The oracle runs on every row, in 128-row chunks over a
thread pool (rows are independent), so whole tensors are compared at every
size.

Acceptance, per element of the compared rows:
  residual     bit-exact;
  y            at most 1 unit in the last place of x's dtype, and a zero y
               with the oracle's sign;
  codes        (FP8 element, NVFP4 / MXFP8 block) bit-exact (signed zeros
               included) where the GPU's y equals the oracle's y bit for bit,
               otherwise at most one code step (MXFP8: in blocks whose scale
               matches), with at most 1e-4 of all codes differing;
  NVFP4 / MXFP8 scales bit-exact in at least 99.99% of blocks (and wherever
               the block's y matches);
  quant step   the GPU's codes and scales equal the oracle's quant step
               applied to the GPU's own y, bit for bit (needs the GPU's y);
  padding      scale-buffer rows >= M and all guard bytes keep the sentinel.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
from fp4_activation_quant_amd import ops

FMT = {torch.bfloat16: O.BF16, torch.float16: O.FP16}
SENTINEL = 0xA5
GUARD = 4096
CODE_DIFF_FRACTION = 1e-4
SCALE_MATCH_FRACTION = 0.9999


def bits16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _guarded(nbytes, dev):
    return torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=dev)


def run_gpu(x, r, w, eps, scale, nvfp4, write_y, device="cuda", misalign=False, norm="gemma",
            quant=True, mxfp8=False):
    """Run the HIP op once on device copies of CPU tensors.  Returns numpy
    outputs and the guard/padding state.  ``misalign`` places x, residual and
    y at a 2-byte offset (a non-16-byte-aligned view).  ``norm`` "plain"
    scales by w instead of 1 + w; ``quant`` False runs add + norm alone (y is
    then always written); ``mxfp8`` selects the MXFP8 output (``nvfp4`` and
    ``scale`` are then ignored and no scale pointer is passed)."""
    mode = ("mxfp8" if mxfp8 else "nvfp4" if nvfp4 else "fp8") if quant else None
    if not quant:
        write_y = True
    if mode != "nvfp4":
        nvfp4 = False
    dev = torch.device(device)
    M, H = x.shape
    dt = x.dtype
    off = 2 if misalign else 0
    act = M * H * 2

    def place(t):
        buf = _guarded(act + off, dev)
        v = buf[off:off + act].view(dt).view(M, H)
        if t is not None:
            v.copy_(t.to(dev))
        return buf, v

    xbuf, xd = place(x)
    rbuf, rd = place(r) if r is not None else (None, None)
    wd = w.to(dev).contiguous()
    sd = torch.tensor([scale], dtype=torch.float32, device=dev)
    qbytes = (M * (H // 2) if nvfp4 else M * H) if quant else 0
    qbuf = _guarded(qbytes + off, dev)
    qv = qbuf[off:off + qbytes]
    if quant:
        qv = qv.view(M, H // 2) if nvfp4 else qv.view(torch.float8_e4m3fn).view(M, H)
    bsn = ops.block_scale_bytes(M, H) if nvfp4 else M * (H // 32) if mode == "mxfp8" else 0
    has_bs = mode in ("nvfp4", "mxfp8")
    bsbuf = _guarded(bsn, dev) if has_bs else None
    ybuf, yd = place(None) if write_y else (None, None)
    if norm == "gemma" and mode in ("fp8", "nvfp4"):
        ops.gemma_add_rms_norm_quant_out(xd, rd, wd, eps, sd, nvfp4, qv,
                                         bsbuf[:bsn] if nvfp4 else None, yd)
    else:
        ops.add_rms_norm_quant_out(xd, rd, wd, eps, sd if mode in ("fp8", "nvfp4") else None, mode,
                                   norm, qv if quant else None, bsbuf[:bsn] if has_bs else None, yd)
    torch.cuda.synchronize(dev)

    def tail_ok(buf, n):
        return bool((buf[off + n:].cpu() == SENTINEL).all()) and bool((buf[:off].cpu() == SENTINEL).all())

    out = {
        "M": M, "H": H, "nvfp4": nvfp4, "dtype": dt, "mode": mode, "norm": norm,
        "x_unchanged": bool(torch.equal(xd.cpu(), x)),
        "residual": bits16(rd) if rd is not None else None,
        "y": bits16(yd) if yd is not None else None,
        "q": (qv.view(torch.uint8).cpu().numpy() if not nvfp4 else qv.cpu().numpy()) if quant else None,
        "bs": bsbuf[:bsn].cpu().numpy() if has_bs else None,
        "guards_ok": all([tail_ok(xbuf, act), tail_ok(qbuf, qbytes),
                          rbuf is None or tail_ok(rbuf, act), ybuf is None or tail_ok(ybuf, act),
                          bsbuf is None or bool((bsbuf[bsn:].cpu() == SENTINEL).all())]),
    }
    return out


def all_rows(M):
    """Every row: the oracle checks whole tensors (on 128-row chunks over a
    thread pool, so the largest workload takes seconds)."""
    return np.arange(M)


def oracle_threads():
    """Host threads for the oracle: the process's CPU affinity, at most 16
    (the host cores a machine typically gives one GPU's process)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def _ord16(b):
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _ord_code(c, sign_bit):
    c = c.astype(np.int64)
    return np.where(c & sign_bit, -(c & (sign_bit - 1)), c & (sign_bit - 1))


def _unpack_e2m1(q):
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)


def gather_scales(bs_flat, rows, H):
    nb = H // 16
    mm, bb = np.meshgrid(rows, np.arange(nb), indexing="ij")
    return bs_flat[O.swizzle_128x4_offset(mm, bb, H)]


CHUNK_ROWS = 128


def _compare_chunk(gpu, xb_all, rb_all, wb, eps, scale, rows, yg_all, fmt):
    """Raw counts for one chunk of rows (aggregated by ``compare``)."""
    M, H, nvfp4 = gpu["M"], gpu["H"], gpu["nvfp4"]
    mode, norm = gpu.get("mode", "nvfp4" if nvfp4 else "fp8"), gpu.get("norm", "gemma")
    xb = xb_all[rows]
    rb = rb_all[rows] if rb_all is not None else None
    ref = O.add_rms_norm_quant(xb, rb, wb, eps, scale, mode, norm, fmt)
    c = {"elements": len(rows) * H}
    if rb is not None:
        c["residual_mismatch"] = int(np.count_nonzero(gpu["residual"][rows] != ref["residual"]))
    y_equal = None
    yg = None
    if yg_all is not None:
        yg = yg_all[rows]
        dy = np.abs(_ord16(yg) - _ord16(ref["y"]))
        c["y_max_ulp"] = int(dy.max()) if dy.size else 0
        c["y_diff"] = int(np.count_nonzero(dy))
        y_equal = yg == ref["y"]
        # +0 and -0 are one ulp step apart in no ordering: count them apart
        c["y_zero_sign_mismatch"] = int(np.count_nonzero((dy == 0) & ~y_equal))
    if mode is None:
        return c
    if mode == "mxfp8":
        cg = gpu["q"][rows]
        cr = ref["q"]
        sg = gpu["bs"].reshape(M, H // 32)[rows]
        sr = ref["scales"]
        c["scale_match"], c["scales"] = int(np.count_nonzero(sg == sr)), int(sr.size)
        same_scale = np.repeat(sg == sr, 32, axis=1)
        step = np.where(same_scale, np.abs(_ord_code(cg, 0x80) - _ord_code(cr, 0x80)), 0)
        c["codes_in_rescaled_blocks"] = int(np.count_nonzero(~same_scale))
        if y_equal is not None:
            blk_eq = y_equal.reshape(len(rows), -1, 32).all(axis=2)
            c["scale_mismatch_where_y_equal"] = int(np.count_nonzero((sg != sr) & blk_eq))
            c["code_mismatch_where_y_equal"] = int(np.count_nonzero(
                (cg != cr).reshape(len(rows), -1, 32).any(axis=2) & blk_eq))
            q2, s2 = O.quant_mxfp8(yg, fmt)
            c["requant_code_mismatch"] = int(np.count_nonzero(q2 != cg))
            c["requant_scale_mismatch"] = int(np.count_nonzero(s2 != sg))
    elif nvfp4:
        cg = _unpack_e2m1(gpu["q"][rows])
        cr = _unpack_e2m1(ref["q"])
        step = np.abs(_ord_code(cg, 8) - _ord_code(cr, 8))
        sg = gather_scales(gpu["bs"], rows, H)
        sr = ref["scales"]
        c["scale_match"], c["scales"] = int(np.count_nonzero(sg == sr)), int(sr.size)
        if y_equal is not None:
            blk_eq = y_equal.reshape(len(rows), -1, 16).all(axis=2)
            c["scale_mismatch_where_y_equal"] = int(np.count_nonzero((sg != sr) & blk_eq))
            c["code_mismatch_where_y_equal"] = int(np.count_nonzero(
                (cg != cr).reshape(len(rows), -1, 16).any(axis=2) & blk_eq))
            q2, s2 = O.quant_nvfp4(yg, fmt, scale)
            c["requant_code_mismatch"] = int(np.count_nonzero(q2 != gpu["q"][rows]))
            c["requant_scale_mismatch"] = int(np.count_nonzero(s2 != sg))
    else:
        cg = gpu["q"][rows]
        cr = ref["q"]
        step = np.abs(_ord_code(cg, 0x80) - _ord_code(cr, 0x80))
        if y_equal is not None:
            c["code_mismatch_where_y_equal"] = int(np.count_nonzero((cg != cr) & y_equal))
            q2 = O.quant_fp8_static(yg, fmt, scale)
            c["requant_code_mismatch"] = int(np.count_nonzero(q2 != cg))
    c["code_max_step"] = int(step.max()) if step.size else 0
    c["code_diff"] = int(np.count_nonzero(cg != cr))
    c["codes"] = int(cg.size)
    return c


_MAX_KEYS = ("y_max_ulp", "code_max_step")


def compare(gpu, x, r, w, eps, scale, rows, y_gpu=None, threads=None):
    """Compare a GPU run with the oracle on ``rows`` (normally every row).
    ``y_gpu`` (full (M, H) uint16) is the GPU's y when the run itself did not
    write it.  The oracle runs on chunks of at most 128 of these rows on a
    thread pool (rows are independent; numpy releases the interpreter lock
    inside its array loops)."""
    M, H, nvfp4 = gpu["M"], gpu["H"], gpu["nvfp4"]
    mode = gpu.get("mode", "nvfp4" if nvfp4 else "fp8")
    fmt = FMT[x.dtype]
    rows = np.asarray(rows, dtype=np.int64)
    xb_all = bits16(x)
    rb_all = bits16(r) if r is not None else None
    wb = bits16(w)
    yg_all = gpu["y"] if gpu["y"] is not None else y_gpu
    chunks = [rows[i:i + CHUNK_ROWS] for i in range(0, len(rows), CHUNK_ROWS)]
    with ThreadPoolExecutor(threads or oracle_threads()) as ex:
        parts = list(ex.map(lambda c: _compare_chunk(gpu, xb_all, rb_all, wb, eps, scale, c, yg_all, fmt),
                            chunks))
    tot = {}
    for p in parts:
        for k, v in p.items():
            tot[k] = max(tot.get(k, 0), v) if k in _MAX_KEYS else tot.get(k, 0) + v
    rep = {"rows": len(rows), "elements": len(rows) * H, "guards_ok": gpu["guards_ok"],
           "x_unchanged": gpu["x_unchanged"]}
    for k in ("residual_mismatch", "y_max_ulp", "y_zero_sign_mismatch", "codes_in_rescaled_blocks",
              "scale_mismatch_where_y_equal", "code_mismatch_where_y_equal", "requant_code_mismatch",
              "requant_scale_mismatch"):
        if k in tot:
            rep[k] = tot[k]
    if "y_diff" in tot:
        rep["y_diff_fraction"] = float(tot["y_diff"] / max(rep["elements"], 1))
    if mode is None:
        rep["code_max_step"] = 0
        rep["code_diff_fraction"] = 0.0
        return rep
    rep["code_max_step"] = tot.get("code_max_step", 0)
    rep["code_diff_fraction"] = float(tot.get("code_diff", 0) / max(tot.get("codes", 0), 1))
    if "scales" in tot:
        rep["scale_match_fraction"] = float(tot["scale_match"] / max(tot["scales"], 1))
    if nvfp4:
        # padding rows of the scale buffer keep the sentinel
        R = O.block_scale_buffer_shape(M, H)[0]
        if R > M:
            pr = gather_scales(gpu["bs"], np.arange(M, R), H)
            rep["padding_written"] = int(np.count_nonzero(pr != SENTINEL))
        else:
            rep["padding_written"] = 0
    return rep


# Whole-tensor figures of the full-size workload comparisons, printed in the
# test run's terminal summary (tests/conftest.py).
SUMMARY = []


def record(name, rep):
    """Keep one line of a passing full-size comparison for the run's summary."""
    parts = [f"{rep['rows']} rows", f"y differs {rep.get('y_diff_fraction', 0.0):.2e} (max {rep.get('y_max_ulp', 0)} ulp)",
             f"codes differ {rep['code_diff_fraction']:.2e} (max {rep['code_max_step']} step)"]
    if "scale_match_fraction" in rep:
        parts.append(f"block scales match {rep['scale_match_fraction']:.6f}")
    parts.append(f"residual mismatches {rep.get('residual_mismatch', 0)}")
    SUMMARY.append(f"{name}: " + ", ".join(parts))


def check(rep):
    """Raise AssertionError listing every bar the report misses."""
    bad = []
    if not rep["guards_ok"]:
        bad.append("wrote outside an output buffer")
    if not rep["x_unchanged"]:
        bad.append("x was modified")
    if rep.get("residual_mismatch", 0):
        bad.append(f"residual mismatches: {rep['residual_mismatch']}")
    if rep.get("y_max_ulp", 0) > 1:
        bad.append(f"y off by {rep['y_max_ulp']} ulp")
    if rep["code_max_step"] > 1:
        bad.append(f"code off by {rep['code_max_step']} steps")
    if rep["code_diff_fraction"] > CODE_DIFF_FRACTION:
        bad.append(f"code diff fraction {rep['code_diff_fraction']:.3g}")
    for k in ("y_zero_sign_mismatch", "code_mismatch_where_y_equal", "scale_mismatch_where_y_equal",
              "requant_code_mismatch", "requant_scale_mismatch", "padding_written"):
        if rep.get(k, 0):
            bad.append(f"{k}: {rep[k]}")
    if "scale_match_fraction" in rep and rep["scale_match_fraction"] < SCALE_MATCH_FRACTION:
        bad.append(f"scale match fraction {rep['scale_match_fraction']:.6f}")
    if bad:
        raise AssertionError("; ".join(bad) + f"  [{rep}]")
    return rep
