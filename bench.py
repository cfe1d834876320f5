"""Benchmark of the fused residual-add + Gemma RMSNorm + quant op on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--eager]

A step is one launch of the whole op (add, norm, y, quant, scale store) over
one batch of the workload, inputs resident in HBM.  The in-place residual
update is part of the op; to keep the residual bounded over many steps the
activation alternates between x and -x from step to step (same work, same
bytes).  Buffer sets (inputs and outputs) rotate from step to step so that at
least 2 GiB of distinct data pass between two uses of a set, which keeps the
256 MB Infinity Cache from serving a step out of the previous ones.  Prints
one JSON line:

  value        whole-job effective HBM GB/s: algorithmic bytes per step x K /
               wall time of the K steps (synchronised on both sides).  The K
               launches are captured once in a HIP graph and the timed region
               is one replay of it (--eager: one Python launch per step);
  roofline     the kernel's duration per launch from HIP events recorded on
               the launch stream: (span of a replay of 2K launches - span of
               a replay of K) / K, each replay queued behind device work so
               no launch waits for the host (eager: one event pair per
               launch); algorithmic bytes / that duration against the 8 TB/s
               HBM peak; traffic = measured HBM bytes per launch
               (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's
               reading) from profiles/traffic.json when it was taken on the
               current kernel source, else null;
  cpu_baseline the CPU oracle timed on a bounded row sample of the same
               workload on this host.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 2 << 30
METRIC = "effective HBM GB/s (and % of peak) + tokens/s for add-RMSNorm+quant, 1 GPU"
KERNEL_SRC_DIR = os.path.join(ROOT, "fp4_activation_quant_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(wl):
    """Bytes the op must move once: reads x, residual, weight and (FP8,
    NVFP4) the scale; writes residual, y, codes and one scale byte per 16
    (NVFP4) or 32 (MXFP8) elements.  Padding rows of the NVFP4 scale buffer
    are not written and not counted."""
    MH = wl.M * wl.H
    rd = 2 * MH + (2 * MH if wl.has_residual else 0) + 2 * wl.H + (0 if wl.mode == "mxfp8" else 4)
    wr = (2 * MH if wl.has_residual else 0) + (2 * MH if wl.write_y else 0)
    wr += {"nvfp4": MH // 2 + MH // 16, "mxfp8": MH + MH // 32, "fp8": MH}[wl.mode]
    return rd, wr


def kernel_sha():
    """Hash of the fused kernel's source files (the shared header, the fused
    kernel template and its per-mode translation units) with comments and
    blank space removed: traffic counters taken on other code are not
    reported, while a comment edit keeps them."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        if name == "gnq_common.hpp" or name.startswith("gnq_fused"):
            h.update(name.encode())
            with open(os.path.join(KERNEL_SRC_DIR, name), encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _code_only(src):
    """C++ source without its comments, one space for each run of blank space
    (the sources hold no string literal with a comment marker in it)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def chunks_per_thread(H, res=False):
    """The fused kernel's 8-element chunks per thread (its launcher's rule)."""
    nchunk = H // 8
    if H <= 4096 or (res and H <= 5120) or (nchunk <= 1024 and nchunk % 256 == 0):
        return 1
    return 2 if nchunk <= 2048 else 4


def fp8_kernel(M, N, K):
    """The FP8 / MXFP8 consumer kernel the library's dispatch picks (16-byte
    aligned scales assumed)."""
    dma = K % 512 == 0
    t256 = -(-M // 256) * -(-N // 256)
    t128 = -(-M // 128) * -(-N // 128)
    if dma and t256 >= 128:
        return "gemm_fp8_tn_dma<256>"
    if dma and (M > 256 or t128 >= 128):
        return "gemm_fp8_tn_dma<128>"
    if M <= 256 and K % 2048 == 0 and K <= 16384:
        return "gemm_fp8_decode"
    if M <= 256 and K % 64 == 0:
        return "gemm_fp8_skinny"
    return "gemm_fp8_tn"


def nvfp4_kernel(M, N, K):
    """The NVFP4 consumer kernel the library's dispatch picks for (M, N, K)."""
    if M <= 8 and M * N <= 12288 and M * (K // 32) * 80 <= 128 * 1024:
        return "gemm_nvfp4_gemv"

    def tiles(mt, nt):
        return -(-M // mt) * -(-N // nt)
    if M > 256 and tiles(256, 256) >= 128:
        return "gemm_nvfp4_big"
    if M >= 128 and tiles(128, 64) >= 192:
        return "gemm_nvfp4_k<4,128,64,4>"
    if M >= 64 and tiles(64, 64) >= 192:
        return "gemm_nvfp4_k<8,64,64,3>"
    if M >= 64 and tiles(64, 32) >= 192:
        return "gemm_nvfp4_k<8,64,32,4>"
    return "gemm_nvfp4_k<8,32,32,4>" if K % 512 == 0 else "gemm_nvfp4_k<4,32,32,8>"


def prefetch_rows(M, H):
    """Whether the fused kernel loops workgroups over the rows, loading the
    next row early (its launcher's rule; 1024 workgroups with two chunks per
    thread, 512 with one)."""
    return 4096 < H < 6144 and 2048 <= M <= 16384


def kernel_name(wl):
    return "fused_rows<{},{},{},{},{}{}>".format(
        wl.dtype, wl.mode, "res" if wl.has_residual else "nores",
        "y" if wl.write_y else "noy", chunks_per_thread(wl.H, wl.has_residual),
        ",prefetch" if prefetch_rows(wl.M, wl.H) else "")


def measured_traffic(wl):
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f).get(wl.name)
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_sha") != kernel_sha():
        return None
    return int(t["fetch_bytes"] + t["write_bytes"])


def cpu_baseline(wl, x, r, w, scale, budget_s):
    """The oracle as it is, on the first rows of the same inputs, until about
    budget_s seconds of CPU work have run (at least 16 rows)."""
    import numpy as np
    import torch
    import oracle as O

    def b16(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    fmt = {"bf16": O.BF16, "fp16": O.FP16}[wl.dtype]
    wb = b16(w)
    chunk = max(1, min(wl.M, (1 << 20) // wl.H))
    rows = 0
    t0 = time.perf_counter()
    while rows < wl.M:
        n = min(chunk, wl.M - rows)
        O.add_rms_norm_quant(b16(x[rows:rows + n]), b16(r[rows:rows + n]) if r is not None else None,
                             wb, wl.eps, scale, wl.mode, "gemma", fmt)
        rows += n
        if time.perf_counter() - t0 >= budget_s and rows >= 16:
            break
    dt = time.perf_counter() - t0
    rd, wr = algorithmic_bytes(wl)
    per_row = (rd + wr - 2 * wl.H - (0 if wl.mode == "mxfp8" else 4)) / wl.M
    out = {"value": round(per_row * rows / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
           "kind": "oracle", "tokens_per_s": round(rows / dt, 1),
           "sample": f"first {rows} of {wl.M} rows of {wl.name}, {dt:.1f} s, numpy single-threaded"}

    # The same oracle calls over row chunks on every host thread the process
    # may use (rows are independent): numpy releases the interpreter lock
    # inside its array loops, so threads run them in parallel.
    threads = host_threads()
    if threads > 1:
        import threading
        from concurrent.futures import ThreadPoolExecutor
        lock = threading.Lock()
        state = {"next": 0, "done": 0}
        t1 = time.perf_counter()

        def worker():
            while True:
                with lock:
                    if state["next"] >= wl.M or time.perf_counter() - t1 >= budget_s:
                        return
                    a = state["next"]
                    state["next"] = min(wl.M, a + chunk)
                b = min(wl.M, a + chunk)
                O.add_rms_norm_quant(b16(x[a:b]), b16(r[a:b]) if r is not None else None,
                                     wb, wl.eps, scale, wl.mode, "gemma", fmt)
                with lock:
                    state["done"] += b - a

        with ThreadPoolExecutor(threads) as ex:
            for f in [ex.submit(worker) for _ in range(threads)]:
                f.result()
        dtp = time.perf_counter() - t1
        n = state["done"]
        out["all_threads"] = {"value": round(per_row * n / dtp / 1e9, 4), "unit": "GB/s",
                              "cores": threads, "tokens_per_s": round(n / dtp, 1),
                              "sample": f"first {n} of {wl.M} rows, {dtp:.1f} s, {threads} threads"}
    return out


def host_threads():
    """Host threads the process may use: its CPU affinity, capped by
    OMP_NUM_THREADS when set."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def copy_calibration(args):
    """Known-size plain copy: each launch reads and writes MIB MiB."""
    import torch
    n = args.copy_calibration << 20
    dev = torch.device("cuda:0")
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": args.steps,
                      "ms_per_copy": round(dt * 1e3, 5), "GBps": round(2 * n / dt / 1e9, 2)}),
          flush=True)


MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 / MXFP8 MFMA
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA


def _time_graph(launch, steps, warmup, stream):
    """Warm up, capture `steps` (and 2 * `steps`) launches in HIP graphs and
    time their replays (_time_graphs); returns (wall seconds of the
    `steps`-launch replay, kernel ms per launch: the differenced figure)."""
    t = _time_graphs(launch, steps, warmup, stream, differenced=True)
    return t["wall_s"], t["diff_ms"]


PAD_BYTES = 1 << 30        # device buffer read ahead of each event-timed replay
PAD_READS = 6              # ~1.5 ms of device work


def _time_graphs(launch, steps, warmup, stream, differenced=False):
    """Warm up, capture `steps` launches (launch(warmup + i)) in one HIP graph
    and, if `differenced`, `2 * steps` launches in a second one; replay each
    once untimed, then time it:

      wall_s    host wall time of a replay of the `steps` launches,
                synchronised on both sides (the bench's timed region);
      span_ms   event span of a replay of the `steps` launches / steps.  The
                replay is queued behind ~1.5 ms of device work (reads of a
                1 GiB pad buffer: reads, so no dirty lines are left to be
                written back while the replay runs) and its start event
                recorded after that work, so every launch of the graph is
                queued before the first one runs: the span holds the
                kernels back to back, with no gap where the device has
                caught up with the host's submission of the graph (such
                gaps, 50-80 us each a few dozen launches into a replay, were
                seen under the profiler);
      diff_ms   (span of the 2 * steps replay - span of the steps replay) /
                steps, both queued the same way: the per-launch time with
                any fixed cost of a replay cancelled, so it does not depend
                on `steps`.
    """
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launch(i)
    torch.cuda.synchronize()
    graphs = []
    for n in ((steps, 2 * steps) if differenced else (steps,)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                launch(warmup + i)
        g.replay()
        torch.cuda.synchronize()
        graphs.append(g)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        graphs[0].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pad = torch.zeros(PAD_BYTES // 4, dtype=torch.int32, device=stream.device)
    torch.cuda.synchronize()
    spans = []
    for k, g in enumerate(graphs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(PAD_READS):
                torch.sum(pad, dtype=torch.int64)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        spans.append(e0.elapsed_time(e1))
    del pad
    out = {"wall_s": wall, "span_ms": spans[0] / steps}
    if differenced:
        out["diff_ms"] = (spans[1] - spans[0]) / steps
    return out


def gemm_cpu_baseline(gw, a, sa, b, sb, budget_s):
    """The oracle GEMM (numpy float64 matmul, one BLAS thread) on the first
    rows of the same operands, until about budget_s seconds."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_limits
    an, bn = a.numpy(), b.numpy()
    rows, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while rows < gw.M:
            if gw.mode == "nvfp4":
                # 128-row chunks: a chunk's block scales are one contiguous
                # slab of the 128x4-tiled buffer (128 x K/16 bytes)
                n = min(128, gw.M - rows)
                slab = sa.numpy()[rows * (gw.K // 16):(rows + 128) * (gw.K // 16)]
                O.gemm_nvfp4(an[rows:rows + n], slab, gw.a_gs, bn, sb.numpy(), gw.b_gs, n, gw.N, gw.K)
                rows += n
                if time.perf_counter() - t0 >= budget_s:
                    break
                continue
            n = min(64, gw.M - rows)
            if gw.mode == "mxfp8":
                O.gemm_mxfp8(an[rows:rows + n], sa[rows:rows + n].numpy(), bn, sb.numpy())
            else:
                O.gemm_fp8_static(an[rows:rows + n], gw.a_scale, bn, gw.b_scale)
            rows += n
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * rows * gw.N * gw.K / dt / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {rows} of {gw.M} rows x all {gw.N} columns of {gw.name}, {dt:.1f} s, "
                      "numpy float64 matmul, one BLAS thread"}


def gemm_main(args):
    """The consumer GEMM: quantized activation x
    quantized weight -> bf16, timed like the op (graph replay, buffer sets
    rotated through >= 2 GiB)."""
    import torch
    from fp4_activation_quant_amd import _lib, ops
    from fp4_activation_quant_amd.workloads import GEMM_WORKLOADS, make_gemm_inputs
    _lib.lib()
    gw = GEMM_WORKLOADS[args.gemm]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# gemm workload {gw.name}: generating inputs", file=sys.stderr, flush=True)
    a, sa, b, sb = make_gemm_inputs(gw)
    M, N, K = gw.M, gw.N, gw.K
    mx = gw.mode == "mxfp8"
    nv = gw.mode == "nvfp4"
    if nv:
        in_bytes = (M + N) * (K // 2) + sa.numel() + sb.numel() + 8
    else:
        in_bytes = M * K + N * K + ((M + N) * (K // 32) if mx else 8)
    out_bytes = 2 * M * N
    n_sets = max(1, min(16, -(-ROTATE_BYTES // (in_bytes + out_bytes))))
    sets = []
    for _ in range(n_sets):
        st = {"a": a.to(dev), "b": b.to(dev), "c": torch.empty((M, N), dtype=torch.bfloat16, device=dev)}
        if mx or nv:
            st["sa"], st["sb"] = sa.to(dev), sb.to(dev)
            if nv:
                st["ga"] = torch.tensor([gw.a_gs], dtype=torch.float32, device=dev)
                st["gb"] = torch.tensor([gw.b_gs], dtype=torch.float32, device=dev)
        else:
            st["sa"] = torch.tensor([gw.a_scale], dtype=torch.float32, device=dev)
            st["sb"] = torch.tensor([gw.b_scale], dtype=torch.float32, device=dev)
        sets.append(st)

    def launch(i):
        st = sets[i % n_sets]
        if nv:
            ops.gemm_nvfp4(st["a"], st["sa"], st["ga"], st["b"], st["sb"], st["gb"], st["c"])
        elif mx:
            ops.gemm_mxfp8(st["a"], st["sa"], st["b"], st["sb"], st["c"])
        else:
            ops.gemm_fp8_static(st["a"], st["sa"], st["b"], st["sb"], st["c"])

    stream = torch.cuda.Stream(device=dev)
    wall, kern_ms = _time_graph(launch, args.steps, args.warmup, stream)
    flop = 2.0 * M * N * K
    ms_per_step = wall * 1e3 / args.steps
    # Bound: whichever of the MFMA time at peak and the HBM time of the
    # operands and output at peak is longer (few activation rows: HBM).
    # the NVFP4 consumer runs the fp16 MFMA on exactly dequantized operands
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if nv else MFMA_FP8_PEAK_TFLOPS
    hbm_bound = (in_bytes + out_bytes) / (HBM_PEAK_GBS * 1e9) > flop / (mfma_peak * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round((in_bytes + out_bytes) / (kern_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flop / (kern_ms * 1e-3) / 1e12, 1),
                "peak": mfma_peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    kernel = nvfp4_kernel(M, N, K) if nv else fp8_kernel(M, N, K)
    out = {
        "metric": "consumer GEMM TFLOP/s (quantized activation x quantized weight -> bf16), 1 GPU",
        "value": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("nvfp4 (e2m1 + e4m3 block scales; fp16 MFMA)" if nv else
                  "mxfp8 (e4m3 + e8m0)" if mx else "e4m3"), "data": "synthetic",
        "config": {"workload": gw.name, "M": M, "N": N, "K": K, "mode": gw.mode,
                   "bytes_in": in_bytes, "bytes_out": out_bytes},
        "launch": "graph", "buffer_sets": n_sets, "kernel_ms": round(kern_ms, 5),
        "roofline": dict(kernel=kernel, **roof),
    }
    out["cpu_baseline"] = (None if args.no_cpu_baseline else
                           gemm_cpu_baseline(gw, a, sa, b, sb, args.cpu_seconds))
    print(json.dumps(out), flush=True)


def chain_main(args):
    """The op feeding the consumer GEMM, fused (add + norm + MXFP8 or NVFP4
    quant, then the GEMM) against unfused (add + norm writing y, the
    standalone quant reading it back, then the GEMM): time per layer input."""
    import torch
    from fp4_activation_quant_amd import _lib, ops
    from fp4_activation_quant_amd.workloads import (WORKLOADS, GEMM_WORKLOADS, make_inputs, make_gemm_inputs,
                                                     load_scale)
    _lib.lib()
    wl = WORKLOADS[args.chain]
    if wl.mode not in ("mxfp8", "nvfp4"):
        raise SystemExit("--chain takes an MXFP8 or NVFP4 workload")
    nv = wl.mode == "nvfp4"
    gw = [g for g in GEMM_WORKLOADS.values() if g.mode == wl.mode and g.M == wl.M and g.K == wl.H][0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, r, w = make_inputs(wl)
    _, _, b, sb = make_gemm_inputs(gw)
    M, H, N = wl.M, wl.H, gw.N
    xd, wd, bd, sbd = x.to(dev), w.to(dev), b.to(dev), sb.to(dev)
    xs = [xd, -xd]
    rd = r.to(dev) if r is not None else None
    y = torch.empty((M, H), dtype=x.dtype, device=dev)
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if nv:
        q = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((ops.round_up(M, 128), ops.round_up(H // 16, 4)), dtype=torch.uint8, device=dev)
        gsd = torch.tensor([load_scale(wl)], dtype=torch.float32, device=dev)
        gbd = torch.tensor([gw.b_gs], dtype=torch.float32, device=dev)
    else:
        q = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
        s = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    res = {}
    for path in ("fused", "unfused"):
        def launch(i, path=path):
            xi = xs[i & 1]
            if nv:
                if path == "fused":
                    ops.add_rms_norm_quant_out(xi, rd, wd, wl.eps, gsd, "nvfp4", "gemma", q, s,
                                               y if wl.write_y else None)
                else:
                    ops.add_rms_norm_quant_out(xi, rd, wd, wl.eps, None, None, "gemma", None, None, y)
                    ops.quant_nvfp4(y, gsd, q, s)
                ops.gemm_nvfp4(q, s, gsd, bd, sbd, gbd, c)
                return
            if path == "fused":
                ops.add_rms_norm_quant_out(xi, rd, wd, wl.eps, None, "mxfp8", "gemma", q, s,
                                           y if wl.write_y else None)
            else:
                ops.add_rms_norm_quant_out(xi, rd, wd, wl.eps, None, None, "gemma", None, None, y)
                ops.quant_mxfp8(y, q, s)
            ops.gemm_mxfp8(q, s, bd, sbd, c)
        stream = torch.cuda.Stream(device=dev)
        wall, kern_ms = _time_graph(launch, args.steps, args.warmup, stream)
        res[path] = kern_ms
    # Row chunks on two streams: the op on chunk j + 1 runs beside the GEMM of
    # chunk j (a memory-bound kernel next to a compute-bound one); every
    # stream stays at the default priority.
    ovl = max(1, args.overlap)
    if ovl > 1 and M % ovl == 0 and not nv:
        rows = M // ovl
        s_norm, s_gemm = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
        done = [torch.cuda.Event() for _ in range(ovl)]

        def launch_ovl(i):
            xi = xs[i & 1]
            cur = torch.cuda.current_stream(dev)
            s_norm.wait_stream(cur)             # fork from the launching (capturing) stream;
            s_gemm.wait_stream(cur)             # the previous step joined it at its end
            for j in range(ovl):
                sl = slice(j * rows, (j + 1) * rows)
                with torch.cuda.stream(s_norm):
                    ops.add_rms_norm_quant_out(xi[sl], rd[sl] if rd is not None else None, wd, wl.eps, None,
                                               "mxfp8", "gemma", q[sl], s[sl], y[sl] if wl.write_y else None)
                    done[j].record(s_norm)
                with torch.cuda.stream(s_gemm):
                    s_gemm.wait_event(done[j])
                    ops.gemm_mxfp8(q[sl], s[sl], bd, sbd, c[sl])
            cur.wait_stream(s_gemm)
            cur.wait_stream(s_norm)

        stream = torch.cuda.Stream(device=dev)
        wall, kern_ms = _time_graph(launch_ovl, args.steps, args.warmup, stream)
        res["fused_overlap"] = kern_ms
    line = {"metric": "norm + quant + consumer GEMM, us per layer input", "workload": wl.name,
            "gemm": gw.name, "fused_us": round(res["fused"] * 1e3, 2),
            "unfused_us": round(res["unfused"] * 1e3, 2),
            "speedup": round(res["unfused"] / res["fused"], 3)}
    if "fused_overlap" in res:
        line.update(overlap_chunks=ovl, fused_overlap_us=round(res["fused_overlap"] * 1e3, 2))
    print(json.dumps(line), flush=True)


def decode_main(args):
    """A decode step at H = N = 4096 (the decode sweep's rows; an FP8
    weight of random finite codes): the op (static FP8) and its consumer
    linear as one fused launch against the two launches (the op, then the
    decode GEMM), per row count.  Weights rotate through >= 2 GiB, so each
    step fetches its weight from HBM as a layer of a real decode step does.
    One JSON line per M: us per step (differenced graph replays queued
    behind device work; the K-launch span / K beside it as a check)."""
    import numpy as np
    import torch
    from fp4_activation_quant_amd import _lib, ops
    from fp4_activation_quant_amd.workloads import WORKLOADS, make_inputs, load_scale
    _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS["fp8_decode_m256_h4096_bf16"]
    x, r, w = make_inputs(wl)
    H = N = wl.H
    s = torch.tensor([load_scale(wl)], dtype=torch.float32, device=dev)
    bs = torch.tensor([0.004], dtype=torch.float32, device=dev)
    rng = np.random.default_rng(9700)
    b0 = (rng.integers(0, 8, size=(N, H)) | (rng.integers(0, 8, size=(N, H)) << 3)
          | (rng.integers(0, 2, size=(N, H)) << 7)).astype(np.uint8)
    n_sets = max(1, ROTATE_BYTES // (N * H))
    bsets = [torch.from_numpy(b0).to(dev) for _ in range(n_sets)]
    wd = w.to(dev)
    for M in [int(v) for v in args.decode.split(",")]:
        xs = [x[:M].to(dev), (-x[:M]).to(dev)]
        rd = r[:M].to(dev)
        rout = torch.empty_like(rd)
        q = torch.empty((M, H), dtype=torch.uint8, device=dev)
        qf = q.view(torch.float8_e4m3fn)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        res = {}
        for path in ("fused", "two_launches"):
            def launch(i, path=path):
                xi, b = xs[(i // n_sets) & 1], bsets[i % n_sets]
                if path == "fused":
                    ops.gemma_add_rms_norm_quant_gemm_fp8_out(xi, rd, rout, wd, wl.eps, s, b, bs, q, None, out)
                else:
                    ops.gemma_add_rms_norm_quant_out(xi, rout, wd, wl.eps, s, False, qf, None, None)
                    ops.gemm_fp8_static(q, s, b, bs, out=out)
            stream = torch.cuda.Stream(device=dev)
            t = _time_graphs(launch, args.steps, args.warmup, stream, differenced=True)
            res[path] = t["diff_ms"] * 1e3
            res[path + "_span"] = t["span_ms"] * 1e3
        print(json.dumps({"metric": "decode step: add + Gemma RMSNorm + FP8 quant + FP8 linear, us per step",
                          "M": M, "H": H, "N": N, "weight_sets": n_sets, "steps": args.steps,
                          "fused_call_runs": "one launch" if M <= 3 else "op + decode GEMM",
                          "fused_us": round(res["fused"], 3), "two_launches_us": round(res["two_launches"], 3),
                          "fused_span_us": round(res["fused_span"], 3),
                          "two_launches_span_us": round(res["two_launches_span"], 3),
                          "speedup": round(res["two_launches"] / res["fused"], 3)}), flush=True)


def block_threads(H, res=False):
    """The fused kernel's workgroup size for rows of H elements (its launch
    rule: chunks per thread, rounded up to whole waves)."""
    nchunk = H // 8
    cpt = chunks_per_thread(H, res)
    return -(-(-(-nchunk // cpt)) // 64) * 64


def traffic_streams(wl):
    """Per-row bytes of the op's read and write streams for a workload: reads
    x (and the residual); writes the residual, y, the codes and the scale
    bytes (NVFP4's last: the probe writes them as a plain row stream, or in
    its tiled form at their 128x4-tiled offsets as the op does)."""
    H = wl.H
    src = [2 * H] + ([2 * H] if wl.has_residual else [])
    dst = ([2 * H] if wl.has_residual else []) + ([2 * H] if wl.write_y else [])
    dst += {"fp8": [H], "nvfp4": [H // 2, H // 16], "mxfp8": [H, H // 32]}[wl.mode]
    return src, dst


def ceiling_main(args):
    """The traffic probe (the op's access structure and byte mix, no
    arithmetic) for each named workload, in several launch forms, timed like
    the op: graph replay, buffer sets rotated through >= 2 GiB, per-launch
    time from the difference of a K- and a 2K-launch replay.  One JSON line
    per workload with every form and the best (the practical ceiling the
    op's figure is compared with).  NVFP4 workloads (M a multiple of 128)
    are also probed with the scale bytes stored at their 128x4-tiled offsets
    in the op's row order, as the op must store them: best_tiled is the best
    of those forms."""
    import torch
    from fp4_activation_quant_amd import _lib
    from fp4_activation_quant_amd.workloads import WORKLOADS
    _lib.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names = list(WORKLOADS) if args.ceiling == "all" else args.ceiling.split(",")
    for name in names:
        wl = WORKLOADS[name]
        src_rb, dst_rb = traffic_streams(wl)
        if any(b % 16 for b in src_rb + dst_rb):
            print(json.dumps({"ceiling": name, "skipped": "row bytes not a multiple of 16"}), flush=True)
            continue
        M = wl.M
        per_launch = M * (sum(src_rb) + sum(dst_rb))
        n_sets = max(1, min(64, -(-ROTATE_BYTES // per_launch)))
        sets = [([torch.ones(M * b // 4, dtype=torch.int32, device=dev) for b in src_rb],
                 [torch.empty(M * b // 4, dtype=torch.int32, device=dev) for b in dst_rb])
                for _ in range(n_sets)]
        op_threads = block_threads(wl.H, wl.has_residual)
        forms = [(op_threads, 0, 0)]
        forms += [(op_threads, g, 1) for g in (256, 512, 768, 1024, 1536, 2048) if g < M]
        forms += [(t, 0, 0) for t in (256, 512, 1024) if t != op_threads and 2 * wl.H <= 64 * t]
        if wl.mode == "nvfp4" and M % 128 == 0:
            forms += [(t, g, f | _lib.NQ_PROBE_TILED_SCALES) for t, g, f in forms]
        stream = torch.cuda.Stream(device=dev)
        results = []
        for threads, grid, pf in forms:
            def launch(i, threads=threads, grid=grid, pf=pf):
                srcs, dsts = sets[i % n_sets]
                st = _lib.nq_traffic_probe([t.data_ptr() for t in srcs], src_rb, [t.data_ptr() for t in dsts],
                                           dst_rb, M, threads, grid, pf, stream.cuda_stream)
                if st != _lib.NQ_OK:
                    raise RuntimeError(f"nq_traffic_probe: status {st}")
            t = _time_graphs(launch, args.steps, args.warmup, stream, differenced=True)
            us = t["diff_ms"] * 1e3
            results.append({"threads": threads, "grid": grid,
                            "prefetch": int(bool(pf & _lib.NQ_PROBE_PREFETCH)),
                            "tiled_scales": int(bool(pf & _lib.NQ_PROBE_TILED_SCALES)), "us": round(us, 3),
                            "GBps": round(per_launch / (us * 1e-6) / 1e9, 1),
                            "span_us": round(t["span_ms"] * 1e3, 3)})
        best = max(results, key=lambda r: r["GBps"])
        line = {"ceiling": name, "bytes_per_launch": per_launch, "rows": M,
                "src_row_bytes": src_rb, "dst_row_bytes": dst_rb, "buffer_sets": n_sets,
                "steps": args.steps, "best_GBps": best["GBps"], "best_us": best["us"],
                "best_frac_of_peak": round(best["GBps"] / HBM_PEAK_GBS, 4)}
        tiled = [r for r in results if r["tiled_scales"]]
        if tiled:
            bt = max(tiled, key=lambda r: r["GBps"])
            line.update(best_tiled_GBps=bt["GBps"], best_tiled_us=bt["us"],
                        best_tiled_frac_of_peak=round(bt["GBps"] / HBM_PEAK_GBS, 4))
        line["forms"] = results
        print(json.dumps(line), flush=True)
        del sets
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused chain instead: add + norm (y to HBM), then the "
                         "standalone quant kernel reading y back (same work, two launches)")
    ap.add_argument("--eager", action="store_true",
                    help="launch step by step from Python instead of replaying the K launches "
                         "captured in one HIP graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the op, time torch's device copy of MIB MiB (the plain "
                         "copy kernel used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--gemm", default=None, metavar="GEMM_WORKLOAD",
                    help="time the consumer GEMM of the quantized activation instead "
                         "(gemm_mxfp8_m8192_n4096_k4096, ...)")
    ap.add_argument("--chain", default=None, metavar="WORKLOAD",
                    help="time the op (MXFP8 output) feeding the consumer GEMM, fused against "
                         "the unfused chain, for a norm workload with a matching GEMM workload")
    ap.add_argument("--write-y", action="store_true",
                    help="also write y for a workload whose default is write_y=False (the "
                         "decode sweep with the normed output, 9H bytes per row)")
    ap.add_argument("--decode", default=None, metavar="ROWS",
                    help="time the fused decode step (op + FP8 linear in one launch) against the two "
                         "launches for these row counts (comma-separated, each <= 8), H = N = 4096")
    ap.add_argument("--ceiling", default=None, metavar="WORKLOADS",
                    help="time the traffic probe (the op's byte mix and access structure, no "
                         "arithmetic) for these workloads (comma-separated, or 'all') instead of the op")
    ap.add_argument("--overlap", type=int, default=1, metavar="CHUNKS",
                    help="with --chain: also time the fused op and the GEMM on row chunks, the op "
                         "of chunk j + 1 on a second stream beside the GEMM of chunk j")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the op is row-independent, and its rows would "
              "split across GPUs with no exchange (--gpus must be 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    from fp4_activation_quant_amd import _lib, ops
    from fp4_activation_quant_amd.workloads import WORKLOADS, DEFAULT_BENCH, make_inputs, load_scale

    if args.copy_calibration:
        return copy_calibration(args)
    if args.gemm:
        return gemm_main(args)
    if args.chain:
        return chain_main(args)
    if args.ceiling:
        return ceiling_main(args)
    if args.decode:
        return decode_main(args)
    _lib.lib()
    wl = WORKLOADS[args.workload or DEFAULT_BENCH]
    if args.write_y and not wl.write_y:
        import dataclasses
        wl = dataclasses.replace(wl, write_y=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# workload {wl.name}: generating inputs", file=sys.stderr, flush=True)
    x, r, w = make_inputs(wl)
    scale = load_scale(wl)
    M, H = wl.M, wl.H
    rbytes, wbytes = algorithmic_bytes(wl)
    total = rbytes + wbytes
    # Buffer sets rotated across steps so that the data a step touches is not
    # left in the 256 MB Infinity Cache by the previous steps: at least
    # ROTATE_BYTES of distinct inputs/outputs per rotation (at most 64 sets).
    n_sets = max(1, min(64, -(-ROTATE_BYTES // total)))
    wd = w.to(dev)
    sd = torch.tensor([scale], dtype=torch.float32, device=dev)
    xp_cpu, xn_cpu = x, -x
    sets = []
    for _ in range(n_sets):
        st = {"x": [xp_cpu.to(dev), xn_cpu.to(dev)],
              "r": r.to(dev) if r is not None else None,
              "y": torch.empty((M, H), dtype=x.dtype, device=dev) if wl.write_y else None}
        if args.unfused and not wl.write_y:
            st["ytmp"] = torch.empty((M, H), dtype=x.dtype, device=dev)
        if wl.nvfp4:
            st["q"] = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
            st["bs"] = torch.empty((ops.round_up(M, 128), ops.round_up(H // 16, 4)),
                                   dtype=torch.uint8, device=dev)
        elif wl.mode == "mxfp8":
            st["q"] = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
            st["bs"] = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
        else:
            st["q"] = torch.empty((M, H), dtype=torch.float8_e4m3fn, device=dev)
            st["bs"] = None
        sets.append(st)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    def launch(i):
        # Set i % n_sets; the activation's sign flips each time a set comes
        # round again, so the in-place residual stays bounded.
        st = sets[i % n_sets]
        xi = st["x"][(i // n_sets) & 1]
        if args.unfused:
            yi = st["y"] if st["y"] is not None else st["ytmp"]
            ops.add_rms_norm_quant_out(xi, st["r"], wd, wl.eps, None, None, "gemma", None, None, yi)
            if wl.nvfp4:
                ops.quant_nvfp4(yi, sd, st["q"], st["bs"])
            elif wl.mode == "mxfp8":
                ops.quant_mxfp8(yi, st["q"], st["bs"])
            else:
                ops.quant_fp8_static(yi, sd, st["q"])
            return
        if wl.mode == "mxfp8":
            ops.add_rms_norm_quant_out(xi, st["r"], wd, wl.eps, None, "mxfp8", "gemma", st["q"],
                                       st["bs"], st["y"])
            return
        ops.gemma_add_rms_norm_quant_out(xi, st["r"], wd, wl.eps, sd, wl.nvfp4, st["q"], st["bs"],
                                         st["y"])

    print(f"# timing {args.steps} steps after {args.warmup} warm-up steps ({n_sets} buffer sets, "
          f"{'graph' if (not args.eager) else 'eager'})", file=sys.stderr, flush=True)
    if not args.eager:
        # The K launches captured once as a HIP graph and replayed: launch
        # overhead off the critical path.  Kernel time per launch = (span of
        # a 2K-launch replay - span of the K-launch replay) / K, both queued
        # behind device work (the K-launch span / K beside it as a check);
        # the host-timed K-launch replay is the timed region of `value`.
        t = _time_graphs(launch, args.steps, args.warmup, stream, differenced=True)
        wall = t["wall_s"]
        kern_ms = [t["diff_ms"]]
        span_ms = t["span_ms"]
    else:
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                launch(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                ev[i][0].record(stream)
                launch(args.warmup + i)
                ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern_ms = [a.elapsed_time(b) for a, b in ev]
        span_ms = None
    kern_ms.sort()
    avg_ms = sum(kern_ms) / len(kern_ms)
    med_ms = kern_ms[len(kern_ms) // 2]

    ms_per_step = wall * 1e3 / args.steps
    value = total / (ms_per_step * 1e-3) / 1e9
    achieved = total / (avg_ms * 1e-3) / 1e9
    traffic = measured_traffic(wl)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "H": H, "act_dtype": wl.dtype,
                   "mode": {"fp8": "fp8_static"}.get(wl.mode, wl.mode), "residual": wl.has_residual,
                   "write_y": wl.write_y, "bytes_per_step": total, "bytes_read": rbytes,
                   "bytes_written": wbytes},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(M / (ms_per_step * 1e-3), 1),
        "launch": "graph" if (not args.eager) else "eager",
        "path": "unfused (2 kernels)" if args.unfused else "fused",
        "buffer_sets": n_sets,
        "kernel_ms": ({"avg": round(avg_ms, 5), "span_per_launch": round(span_ms, 5),
                       "method": "(span of a 2K-launch graph replay - span of a K-launch replay) / K, each "
                                 "replay queued behind device work; span_per_launch = the K-launch span / K"}
                      if span_ms is not None else
                      {"avg": round(avg_ms, 5), "median": round(med_ms, 5), "min": round(kern_ms[0], 5),
                       "max": round(kern_ms[-1], 5), "method": "event pair per eager launch"}),
        "roofline": {"bound": "hbm", "kernel": kernel_name(wl), "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, x, r, w, scale, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
