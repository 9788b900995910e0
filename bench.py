#!/usr/bin/env python3
"""Throughput of the fused gate-up SwiGLU on one MI355X.

A step is one pass of the hot path over one batch: the forward
y = silu(g) * u followed by the out-of-place backward [dgate | dup], on the
wide-FFN workload x [S=2048, B=4, 2n] with n = 32768 in bf16 (8192 tokens x
65536 columns), inputs resident in HBM before the timed region. The value is
algorithmic bytes per step (forward 3 and backward 5 element-sizes per
(row, column) pair: 8 * 2 B * 8192 * 32768 = 4.295 GB) over the measured
step time (K steps of back-to-back launches between two synchronisations),
in GB/s (1e9 B/s).

Also measured in the same run: each kernel's own time from HIP events on the
stream it runs on (forward and backward in a second timed region of K steps,
and the in-place backward), a plain copy of the same size as the backward's
traffic for context, and the CPU oracle on a bounded sample of the same
workload (the cpu_baseline).

One JSON line goes to stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused SwiGLU fwd+bwd achieved HBM GB/s (and % of peak) at S=2048,B=4,n=32768 bf16"
PEAK_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
CALIB_BYTES = 1 << 30
# Sources of the forward and backward kernels timed here (the traffic record
# is only used while they are unchanged).
KERNEL_SRCS = [os.path.join(ROOT, "swiglu_activation_amd", "csrc", f)
               for f in ("swiglu_gateup.hip", "swiglu_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "swiglu_bwd_wide_bf16_n32768_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per backward launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on another kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^kernel_source_sha256_16:\s*(\w+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not t or m.group(1) != source_digest():
        return None
    return float(t.group(1))


def cpu_baseline(w, x_h, dy_h, seconds: float, outputs=None):
    """The oracle as it stands, in one process, on a bounded sample of the
    workload: consecutive 512-row blocks from row 0 until about `seconds` of
    CPU time is spent in it (or the rows run out).

    outputs: optionally the GPU's y and dx of the timed step, as stored
    ([rows, n] and [rows, 2n]; bf16 as bit patterns). The oracle's values of
    the sampled rows are then also compared with them, outside the timed
    part: bf16 by ulp distance to the correctly rounded value, fp32 by
    relative error."""
    import numpy as np

    import oracle
    rows = 0
    dt = 0.0
    worst = {"fwd": 0.0, "bwd": 0.0}
    over = 0
    while rows < w.rows and dt < seconds:
        r1 = min(rows + 512, w.rows)
        t0 = time.perf_counter()
        xf = oracle.widen(x_h[rows:r1], w.dtype)
        dyf = oracle.widen(dy_h[rows:r1], w.dtype)
        y = oracle.oracle_fwd(xf)
        dx = oracle.oracle_bwd(xf, dyf)
        dt += time.perf_counter() - t0
        assert y.shape == (r1 - rows, w.n) and dx.shape == (r1 - rows, 2 * w.n)
        if outputs is not None:
            for what, got, ref in (("fwd", outputs[0][rows:r1], y), ("bwd", outputs[1][rows:r1], dx)):
                if w.dtype == "bf16":
                    d = oracle.bf16_ulp_distance(got, oracle.round_f64_to_bf16_bits(ref))
                    over += int(np.count_nonzero(d > 2))
                else:
                    g = np.asarray(got, dtype=np.float64)
                    d = np.abs(g - ref) / np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
                worst[what] = max(worst[what], float(d.max()))
        rows = r1
    bytes_ = 8 * w.elem_bytes * rows * w.n
    parity = None
    if outputs is not None:
        if w.dtype == "bf16":
            parity = {"rows": rows, "elements": 3 * rows * w.n, "max_ulp_fwd": int(worst["fwd"]),
                      "max_ulp_bwd": int(worst["bwd"]), "over_2_ulp": over}
        else:
            parity = {"rows": rows, "elements": 3 * rows * w.n, "max_rel_fwd": worst["fwd"],
                      "max_rel_bwd": worst["bwd"]}
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"rows 0..{rows} of {w.rows} ({rows * w.n} gate/up pairs) of {w.name}: "
                      "widen to float64, forward, backward (numpy, one thread)",
            "timed_outputs_vs_oracle": parity,
            "all_cores": cpu_baseline_all_cores(w, x_h, dy_h),
            "other_rows": cpu_baseline_other_rows(w, x_h, dy_h)}


def cpu_baseline_all_cores(w, x_h, dy_h, block: int = 32, max_threads: int = 16):
    """The same oracle over the whole workload, split by row blocks over a
    pool of threads, one per core this process may run on (at most
    `max_threads`). numpy drops the GIL inside its array loops, so the blocks
    run in parallel; threads rather than processes keep the GPU-initialised
    process from being forked."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    threads = max(1, min(len(os.sched_getaffinity(0)), max_threads))

    def one(r0):
        r1 = min(r0 + block, w.rows)
        xf = oracle.widen(x_h[r0:r1], w.dtype)
        dyf = oracle.widen(dy_h[r0:r1], w.dtype)
        y = oracle.oracle_fwd(xf)
        dx = oracle.oracle_bwd(xf, dyf)
        return y.shape == (r1 - r0, w.n) and dx.shape == (r1 - r0, 2 * w.n)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as pool:
        ok = all(pool.map(one, range(0, w.rows, block)))
    dt = time.perf_counter() - t0
    assert ok
    return {"value": round(8 * w.elem_bytes * w.rows * w.n / dt / 1e9, 4), "unit": "GB/s",
            "cores": threads, "seconds": round(dt, 3),
            "sample": f"all {w.rows} rows of {w.name}, {block}-row blocks over {threads} threads"}


def cpu_baseline_other_rows(w, x_h, dy_h, rows: int = 512):
    """The oracle of the bias / per-token-scale variants and of the fc1
    projection with the SwiGLU epilogue, each on a small bounded sample and
    one thread (float64 matmuls limited to one BLAS thread), as the CPU
    figure beside those rows' GPU legs."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    out = {}
    rows = min(rows, w.rows)
    rng = np.random.default_rng(w.seed)
    with threadpool_limits(limits=1):
        # bias + scale: forward and backward (dx, dbias, dscale) on `rows` rows
        xf = oracle.widen(x_h[:rows], w.dtype)
        dyf = oracle.widen(dy_h[:rows], w.dtype)
        bias = rng.standard_normal(2 * w.n) * 0.5
        scale = rng.uniform(0.05, 1.0, rows)
        t0 = time.perf_counter()
        oracle.oracle_fwd_bias_scale(xf, bias, scale)
        oracle.oracle_bwd_bias_scale(xf, dyf, bias, scale)
        dt = time.perf_counter() - t0
        out["bias_scale"] = {"value": round(8 * w.elem_bytes * rows * w.n / dt / 1e9, 4),
                             "unit": "GB/s (base op's bytes)", "cores": 1, "seconds": round(dt, 3),
                             "sample": f"rows 0..{rows} of {w.name} with a bias and a scale"}
        # fc1 + SwiGLU: 64 tokens against the full weights of hidden 4096, n 4096
        m, k, n = 64, 4096, 4096
        a = rng.standard_normal((m, k))
        wt = rng.standard_normal((2 * n, k)) / np.sqrt(k)
        t0 = time.perf_counter()
        y = oracle.oracle_fc1_swiglu(a, wt)
        dt = time.perf_counter() - t0
        assert y.shape == (m, n)
        out["fc1_swiglu"] = {"value": round(2.0 * m * k * 2 * n / dt / 1e12, 6),
                             "unit": "TFLOP/s", "cores": 1, "seconds": round(dt, 3),
                             "sample": f"{m} tokens x hidden {k} x n {n} (float64)"}
    return out


PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak


def pair_times(stream, f1, f2, iters: int, warm_s: float = 0.1, between=None):
    """Medians of pair_samples (ms)."""
    import numpy as np
    t1, t2 = pair_samples(stream, f1, f2, iters, warm_s, between)
    return float(np.median(t1)), float(np.median(t2))


def pair_samples(stream, f1, f2, iters: int, warm_s: float = 0.1, between=None):
    """Event times (ms) of f1 and of f2, pair by pair, run alternately back to back
    on `stream`: untimed pairs for `warm_s` seconds first (the first few
    milliseconds of a new load can run up to 15 % slow while the clocks
    settle), then `iters` timed pairs with one synchronisation at the end, so
    the GPU never idles between launches. `between` (untimed) runs before
    each timed call, e.g. to leave the caches in the same state for both."""
    import torch
    t_end = time.perf_counter() + warm_s
    while True:
        for _ in range(4):
            f1()
            f2()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    ev = []
    for _ in range(iters):
        a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        if between is not None:
            between()
        a.record(stream)
        f1()
        b.record(stream)
        if between is not None:
            between()
        c.record(stream)
        f2()
        d.record(stream)
        ev.append((a, b, c, d))
    ev[-1][3].synchronize()
    t = [(a.elapsed_time(b), c.elapsed_time(d)) for a, b, c, d in ev]
    return [x[0] for x in t], [x[1] for x in t]


def hbm_roofline(kernel: str, bytes_: float, ms: float) -> dict:
    """Roofline object of an HBM-bound kernel: algorithmic bytes over its
    average event-timed launch, against the 8 TB/s peak."""
    achieved = bytes_ / ms / 1e6
    return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4), "bytes_per_launch": bytes_}


def fc1_leg(dev, stream, tokens: int, shapes=((4096, 4096), (8192, 32768)), iters: int = 25,
            clock_warmup_s: float = 0.3):
    """fc1 projection with the SwiGLU epilogue (one kernel) against
    torch.matmul (hipBLASLt) followed by the elementwise SwiGLU, for
    (hidden, n) pairs at the given token count; 2 m k 2n FLOPs."""
    import numpy as np
    import torch

    import swiglu_activation_amd as sw
    out = {}
    for si, (hidden, n) in enumerate(shapes):
        gen = torch.Generator(device=dev).manual_seed(hidden + n)
        a = torch.randn(tokens, hidden, device=dev, generator=gen).bfloat16()
        wt = (torch.randn(2 * n, hidden, device=dev, generator=gen) / hidden ** 0.5).bfloat16()
        y = torch.empty(tokens, n, dtype=torch.bfloat16, device=dev)
        xbuf = torch.empty(tokens, 2 * n, dtype=torch.bfloat16, device=dev)
        flops = 2.0 * tokens * hidden * 2 * n

        if si == 0:
            # Untimed: sustained matrix-core load until the clocks have
            # settled (a few launches are not enough; the first ~100 ms of
            # such work run slower).
            t_end = time.perf_counter() + clock_warmup_s
            while time.perf_counter() < t_end:
                for _ in range(8):
                    sw.swiglu_fc1_fwd(a, wt, y)
                torch.cuda.synchronize()
        # Each comparison alternates its two sides launch by launch, so both
        # see the same clocks (which drift by several percent over seconds
        # of matrix-core load); medians over the pairs. Before each timed
        # launch, 512 MiB are written (untimed), which evicts the 256 MiB
        # Infinity Cache: both sides start with their inputs in HBM, as after
        # the other layers of a model, instead of one side finding what the
        # other left behind.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = flush.zero_
        tf, tu = pair_samples(
            stream, lambda: sw.swiglu_fc1_fwd(a, wt, y),
            lambda: (torch.matmul(a, wt.t(), out=xbuf), sw.swiglu_gateup_fwd(xbuf, y)), iters,
            between=cold)
        tfx, tm = pair_samples(stream, lambda: sw.swiglu_fc1_fwd(a, wt, y, x_out=xbuf),
                               lambda: torch.matmul(a, wt.t(), out=xbuf), iters, between=cold)
        del flush
        med = lambda v: float(np.median(v))
        fused, unfused, fused_x, mm = med(tf), med(tu), med(tfx), med(tm)

        def warm(fn, reps=10):
            # back to back with itself, so its inputs stay in the caches
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            e1.synchronize()
            return e0.elapsed_time(e1) / reps

        fused_warm = warm(lambda: sw.swiglu_fc1_fwd(a, wt, y))
        unfused_warm = warm(lambda: (torch.matmul(a, wt.t(), out=xbuf), sw.swiglu_gateup_fwd(xbuf, y)))
        # the clocks move by up to 30 % over tens of milliseconds: the ratio
        # within each pair is the steadier comparison
        ratio = med([f / u for f, u in zip(tf, tu)])
        ratio_x = med([f / u for f, u in zip(tfx, tm)])
        out[f"tokens{tokens}_hidden{hidden}_n{n}"] = {
            "roofline": {"bound": "mfma", "kernel": "swiglu_fc1_kernel",
                         "achieved": round(flops / fused / 1e9, 1), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(flops / fused / 1e9 / PEAK_BF16_TFLOPS, 4),
                         "flops_per_launch": flops},
            "fused_ms": round(fused, 4), "fused_TFLOPs": round(flops / fused / 1e9, 1),
            "fused_frac_of_peak": round(flops / fused / 1e9 / PEAK_BF16_TFLOPS, 4),
            "fused_with_x_ms": round(fused_x, 4),
            "hipblaslt_matmul_ms": round(mm, 4),
            "hipblaslt_TFLOPs": round(flops / mm / 1e9, 1),
            "matmul_then_swiglu_ms": round(unfused, 4),
            "fused_over_matmul_then_swiglu": round(ratio, 4),
            "warm": {"fused_ms": round(fused_warm, 4), "matmul_then_swiglu_ms": round(unfused_warm, 4),
                     "note": "each launched back to back with itself, inputs left in the caches"},
            "fused_with_x_over_matmul": round(ratio_x, 4),
            "pairs": iters}
        log(f"[bench] fc1 h={hidden} n={n}: fused {fused:.3f} ms ({flops / fused / 1e9:.0f} TFLOP/s), "
            f"matmul {mm:.3f} ms, matmul+swiglu {unfused:.3f} ms (per-pair ratio {ratio:.3f}); "
            f"warm: fused {fused_warm:.3f} ms, matmul+swiglu {unfused_warm:.3f} ms")
        del a, wt, y, xbuf
    return out


def bias_scale_leg(dev, stream, w, x, dy, y, dx, iters: int = 20):
    """Bias + per-token scale variants on the workload's tensors: forward,
    and backward with dx, dbias and dscale (the reductions included)."""
    import torch

    import swiglu_activation_amd as sw
    tdt = x.dtype
    e = w.elem_bytes
    fwd_bytes, bwd_bytes = 3 * e * w.rows * w.n, 5 * e * w.rows * w.n
    gen = torch.Generator(device=dev).manual_seed(w.seed)
    bias_t = (torch.randn(2 * w.n, device=dev, generator=gen) * 0.5).to(tdt)
    scale_t = torch.rand(w.shape[:-1], device=dev, generator=gen) * 0.95 + 0.05
    ws = torch.empty(sw.swiglu_gateup_bias_scale_workspace_size(w.rows, w.n, True, True),
                     dtype=torch.uint8, device=dev)
    bf, bb = pair_times(stream, lambda: sw.swiglu_gateup_bias_scale_fwd(x, bias_t, scale_t, y),
                        lambda: sw.swiglu_gateup_bias_scale_bwd(dy, x, bias_t, scale_t, dx,
                                                                workspace=ws), iters)
    # the routed-expert form: a per-token scale and no bias, dx and dscale
    sf, sb = pair_times(stream, lambda: sw.swiglu_gateup_bias_scale_fwd(x, None, scale_t, y),
                        lambda: sw.swiglu_gateup_bias_scale_bwd(dy, x, None, scale_t, dx,
                                                                workspace=ws), iters)
    # algorithmic bytes: the base op's, plus one read of the bias row and the
    # scales, plus the fp32 dbias and dscale written by the backward
    extra_in = 2 * w.n * e + 4 * w.rows
    fwd_alg, bwd_alg = fwd_bytes + extra_in, bwd_bytes + extra_in + 4 * 2 * w.n + 4 * w.rows
    return {"fwd_ms": round(bf, 5), "bwd_ms": round(bb, 5),
            "roofline_fwd": hbm_roofline("swiglu_fwd_bs_kernel (bias, scale)", fwd_alg, bf),
            "roofline_bwd": hbm_roofline("swiglu_bwd_bs_tile_kernel + sums (dx, dbias, dscale)",
                                         bwd_alg, bb),
            "fwd_GBps": round(fwd_bytes / bf / 1e6, 1),
            "bwd_GBps": round(bwd_bytes / bb / 1e6, 1),
            "what": "z = x + bias, y = s * silu(z_g) * z_u; bwd writes dx, dbias, "
                    "dscale (GB/s on the base op's bytes)",
            "scale_only": {"fwd_ms": round(sf, 5), "bwd_ms": round(sb, 5),
                           "roofline_fwd": hbm_roofline("swiglu_fwd_bs_kernel (scale)",
                                                        fwd_bytes + 4 * w.rows, sf),
                           "roofline_bwd": hbm_roofline("swiglu_bwd_bs1_kernel + sum (dx, dscale)",
                                                        bwd_bytes + 8 * w.rows, sb),
                           "fwd_GBps": round(fwd_bytes / sf / 1e6, 1),
                           "bwd_GBps": round(bwd_bytes / sb / 1e6, 1),
                           "what": "no bias, per-token scale; bwd writes dx and dscale"}}


def configs_leg(dev, stream, names, replays: int = 20, parity_rows: int = 512):
    """Every other workload's forward and backward (in place where the
    workload says so), as context for the headline: device-drawn inputs of
    the workload's shape and dtype (timing does not depend on the values),
    rotated over enough buffer sets that each launch reads data last touched
    more than 512 MB earlier, so the 256 MB Infinity Cache cannot serve it.
    The launches over all sets are captured in one HIP graph per pass and the
    graph is replayed, so host launch overhead does not show in the times of
    the short kernels (these workloads run 2 to 420 us per launch). A graph
    holds at least 32 launches; each figure is the per-launch time, median
    over `replays` replays, with the min and max.

    The last `parity_rows` rows of the first set hold the workload's own
    recipe (synth), and the timed launches' outputs of those rows are kept
    (the in-place backward's input rows are restored before its last replay),
    for the oracle comparison in the CPU-baseline leg.

    Beside each pass, a zero-arithmetic stream of the same bytes (one-shot
    grid of 256 lanes over separate flat streams, same rotation and graph
    replay) gives what the memory system allows at that size."""
    import numpy as np
    import torch

    import ceiling
    import synth
    import swiglu_activation_amd as sw
    out, samples = {}, {}
    for name in names:
        w = synth.WORKLOADS[name]
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        e = w.elem_bytes
        fwd_bytes, bwd_bytes = 3 * e * w.rows * w.n, 5 * e * w.rows * w.n
        # (at most 64 sets: the tiny workload is bound by launch latency anyway)
        sets = min(64, max(2, -(-(512 << 20) // fwd_bytes) + 1))
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        bufs = []
        for _ in range(sets):
            x = torch.randn(w.shape, device=dev, generator=gen).to(tdt)
            dy = torch.randn(w.shape[:-1] + (w.n,), device=dev, generator=gen).to(tdt)
            y = torch.empty(w.shape[:-1] + (w.n,), dtype=tdt, device=dev)
            dx = None if w.in_place else torch.empty_like(x)
            bufs.append((x, dy, y, dx))
        r0 = max(0, w.rows - parity_rows)
        xs_h, dys_h = synth.make_x(w, r0, w.rows), synth.make_dy(w, r0, w.rows)

        def dev_rows(a):
            if w.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        def host_rows(t, cols):
            a = t.reshape(w.rows, cols)[r0:]
            if w.dtype == "bf16":
                return a.view(torch.int16).cpu().numpy().view(np.uint16)
            return a.cpu().numpy()

        x0_rows = bufs[0][0].view(w.rows, 2 * w.n)[r0:]
        x0_rows.copy_(dev_rows(xs_h))
        bufs[0][1].view(w.rows, w.n)[r0:].copy_(dev_rows(dys_h))
        torch.cuda.synchronize()

        # Launch order of one graph: at least 32 launches cycling over sets
        # 1.. (each set's data last touched more than 512 MB earlier), then
        # set 0, which holds the sampled rows, once, last.
        order = [1 + i % (sets - 1) for i in range(max(sets - 1, 32))] + [0]

        def fwd_pass():
            for i in order:
                x, dy, y, dx = bufs[i]
                sw.swiglu_gateup_fwd(x, y)

        def bwd_pass():
            for i in order:
                x, dy, y, dx = bufs[i]
                if w.in_place:
                    sw.swiglu_gateup_bwd(dy, x, in_place=True)
                else:
                    sw.swiglu_gateup_bwd(dy, x, dx)

        def replayed(fn, before_last=None):
            fn()                                              # warm up outside the graph
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for i in range(replays):
                if before_last is not None and i == replays - 1:
                    before_last()
                    torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                b.synchronize()
                ts.append(a.elapsed_time(b) / len(order))
            del g
            return float(np.median(ts)), min(ts), max(ts)

        res = {}
        sample = {"rows": [r0, w.rows], "x": xs_h, "dy": dys_h}
        for pname, fn, nbytes in (("fwd", fwd_pass, fwd_bytes), ("bwd", bwd_pass, bwd_bytes)):
            restore = (lambda: x0_rows.copy_(dev_rows(xs_h))) if (w.in_place and pname == "bwd") \
                else None
            t, tmin, tmax = replayed(fn, restore)
            res[f"{pname}_us"] = round(t * 1e3, 2)
            res[f"{pname}_us_min_max"] = [round(tmin * 1e3, 2), round(tmax * 1e3, 2)]
            res[f"{pname}_GBps"] = round(nbytes / t / 1e6, 1)
            if pname == "fwd":
                sample["y"] = host_rows(bufs[0][2], w.n)
            else:
                sample["dx"] = host_rows(bufs[0][0] if w.in_place else bufs[0][3], 2 * w.n)
        del bufs
        # the same bytes with no arithmetic, independent structure
        if (w.n * e) % 16 == 0:
            nvec = w.rows * w.n * e // 16
            fsets = [ceiling.FlatStreams(nvec, dev) for _ in range(sets)]
            for pname, mix, nbytes in (("fwd", "fwd", fwd_bytes), ("bwd", "bwd", bwd_bytes)):
                t, _, _ = replayed(lambda: [ceiling.probe(0, mix, fsets[i]) for i in order])
                res[f"ceiling_{pname}_GBps"] = round(nbytes / t / 1e6, 1)
                res[f"{pname}_frac_of_ceiling"] = round(res[f"{pname}_GBps"] / (nbytes / t / 1e6), 4)
            del fsets
        res.update({"bwd": "in place" if w.in_place else "out of place", "buffer_sets": sets,
                    "timing": f"HIP graph of {len(order)} launches cycling over the buffer sets, "
                              f"median of {replays} replays"})
        out[w.name] = res
        samples[w.name] = sample
    return out, samples


def ceiling_leg(dev, stream, w, x, dy, y, dx, fwd_ms: float, bwd_ms: float, batches: int = 10,
                per_batch: int = 5):
    """Zero-arithmetic streaming ceilings at the headline size: the row-packed
    patterns on the workload's own buffers, and every independent structure
    (ceiling.STRUCTURES) on separate flat streams of the same bytes, for the
    forward and backward mixes and for read-only, write-only and copy
    traffic. Median over `batches` batches of `per_batch` back-to-back
    launches. The SwiGLU kernels' times are set against the best of all."""
    import numpy as np
    import torch

    import ceiling
    e = w.elem_bytes
    nv16 = w.n * e // 16
    nvec = w.rows * nv16

    def timed(fn):
        fn()
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(batches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(per_batch):
                fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) / per_batch)
        return float(np.median(ts))

    res = {"row_packed": {}, "independent": {}}
    for pattern, mix, out in ((0, "fwd", y), (1, "bwd", dx)):
        t = timed(lambda: ceiling.launch(pattern, x, dy, out, w.rows, nv16, stream))
        res["row_packed"][mix] = {"ms": round(t, 5),
                                  "GBps": round(ceiling.mix_bytes(mix, nvec) / t / 1e6, 1)}
    fs = ceiling.FlatStreams(nvec, dev)
    for mix in ceiling.MIXES:
        res["independent"][mix] = {}
        for s, sname in ceiling.STRUCTURES.items():
            t = timed(lambda: ceiling.probe(s, mix, fs, stream))
            res["independent"][mix][sname] = round(ceiling.mix_bytes(mix, nvec) / t / 1e6, 1)
    del fs
    best = {}
    for mix, kernel_ms in (("fwd", fwd_ms), ("bwd", bwd_ms)):
        cands = dict(res["independent"][mix])
        cands["row-packed (the SwiGLU kernels' structure)"] = res["row_packed"][mix]["GBps"]
        sname = max(cands, key=cands.get)
        kernel_gbps = ceiling.mix_bytes(mix, nvec) / kernel_ms / 1e6
        ind = max(res["independent"][mix], key=res["independent"][mix].get)
        best[mix] = {"best_structure": sname, "GBps": cands[sname],
                     "best_independent_structure": ind,
                     "best_independent_GBps": res["independent"][mix][ind],
                     "kernel_GBps": round(kernel_gbps, 1),
                     "kernel_frac_of_best": round(kernel_gbps / cands[sname], 4)}
    res["best"] = best
    return res


def oracle_parity(dtype: str, got, ref, den=None) -> dict:
    """Stored GPU outputs (float32 values, or bf16 bit patterns) against
    float64 oracle values: bf16 by ulp distance to the correctly rounded value
    (bar 2), fp32 by relative error (bar 1e-5; where the reference is 0 the
    output must be 0). den: for dgate, the scale |dy u sigma| (1 + |g| (1 -
    sigma)) of the scale-aware error, reported beside the bar, not gated."""
    import numpy as np

    import oracle
    st = {"elements": int(ref.size)}
    if dtype == "bf16":
        d = oracle.bf16_ulp_distance(got, oracle.round_f64_to_bf16_bits(ref))
        st.update({"max_ulp": int(d.max()) if d.size else 0,
                   "over_2_ulp": int(np.count_nonzero(d > 2))})
        g = oracle.bf16_bits_to_f64(got)
    else:
        g = np.asarray(got, dtype=np.float64)
        nz = ref != 0
        rel = np.abs(g - ref)[nz] / np.abs(ref[nz])
        st.update({"max_rel": float(rel.max()) if rel.size else 0.0,
                   "over_1e-5": int(np.count_nonzero(rel > 1e-5)) +
                   int(np.count_nonzero((~nz) & (g != 0)))})
    if den is not None:
        m = den > 0
        st["max_scale_aware"] = float((np.abs(g - ref)[m] / den[m]).max()) if m.any() else 0.0
    return st


def oracle_parity_of_sample(dtype: str, n: int, s: dict) -> dict:
    """Per-pass parity of one sample of timed outputs (configs leg)."""
    import numpy as np

    import oracle
    xf, dyf = oracle.widen(s["x"], dtype), oracle.widen(s["dy"], dtype)
    y_ref, dx_ref = oracle.oracle_fwd(xf), oracle.oracle_bwd(xf, dyf)
    g, u = xf[:, :n], xf[:, n:]
    sig = oracle.sigmoid(g)
    den = np.abs(dyf * u * sig) * (1.0 + np.abs(g) * (1.0 - sig))
    return {"rows": s["rows"],
            "fwd": oracle_parity(dtype, s["y"], y_ref),
            "bwd_dgate": oracle_parity(dtype, s["dx"][:, :n], dx_ref[:, :n], den),
            "bwd_dup": oracle_parity(dtype, s["dx"][:, n:], dx_ref[:, n:])}


def calib_copies(dev):
    """Known-size plain copies, each reading and writing exactly CALIB_BYTES
    (torch copy_ and an elementwise negation): the byte-counter calibration
    for rocprofv3 --pmc runs."""
    import torch
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    log(f"[bench] calibration copies of {CALIB_BYTES} bytes done")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="synthetic workload name")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time bound of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the fwd+bwd step (for profiling runs)")
    ap.add_argument("--fc1-only", action="store_true",
                    help="time only the fc1 projection with the SwiGLU epilogue, print its "
                         "figures as one JSON line, and exit (for profiling runs)")
    ap.add_argument("--bias-scale-only", action="store_true",
                    help="time only the bias / per-token-scale forward and backward on the "
                         "workload, print their figures as one JSON line, and exit")
    ap.add_argument("--configs-only", action="store_true",
                    help="time only the other workloads' forward and backward (rotated buffers, "
                         "graph replay): the one named by --workload, else all but the headline; "
                         "print their figures as one JSON line, and exit (for profiling runs)")
    ap.add_argument("--calib", action="store_true",
                    help="also run plain 1 GiB copies (torch copy_ and an elementwise "
                         "negation) as the byte-counter calibration for rocprofv3 --pmc")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported. The op is "
              "elementwise and shards with no communication, so N GPUs each run this "
              "single-GPU workload on their own shard.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import swiglu_activation_amd as sw

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    if not os.path.exists(sw.library_path()):
        from swiglu_activation_amd import build
        build.build()
    sw.load_library()

    w = synth.WORKLOADS[args.workload or synth.HEADLINE]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.fc1_only:
        res = fc1_leg(dev, torch.cuda.current_stream(dev), w.rows, iters=args.steps)
        print(json.dumps({"fc1_swiglu": res}), flush=True)
        return
    if args.configs_only:
        names = [args.workload] if args.workload else [k for k in synth.WORKLOADS if k != synth.HEADLINE]
        res, _ = configs_leg(dev, torch.cuda.current_stream(dev), names)
        if args.calib:
            calib_copies(dev)
        print(json.dumps({"other_workloads": res}), flush=True)
        return
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    log(f"[bench] workload {w.name}: x {w.shape} {w.dtype}; drawing inputs")
    x_h, dy_h = synth.make_x(w), synth.make_dy(w)

    def up(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x = up(x_h).reshape(w.shape)
    dy = up(dy_h).reshape(w.shape[:-1] + (w.n,))
    y = torch.empty(w.shape[:-1] + (w.n,), dtype=tdt, device=dev)
    dx = torch.empty(w.shape, dtype=tdt, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.bias_scale_only:
        res = bias_scale_leg(dev, stream, w, x, dy, y, dx, iters=args.steps)
        if args.calib:
            calib_copies(dev)
        print(json.dumps({"bias_scale": res}), flush=True)
        return

    e = w.elem_bytes
    pairs = w.rows * w.n
    fwd_bytes, bwd_bytes = 3 * e * pairs, 5 * e * pairs
    step_bytes = fwd_bytes + bwd_bytes

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        sw.swiglu_gateup_fwd(x, y)
        sw.swiglu_gateup_bwd(dy, x, dx)
    torch.cuda.synchronize()

    K = args.steps
    # Timed region 1, the value: K steps of plain back-to-back launches,
    # bracketed by synchronisations, with nothing else on the stream (HIP
    # events recorded between the launches cost about 11 us per step).
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        sw.swiglu_gateup_fwd(x, y)
        sw.swiglu_gateup_bwd(dy, x, dx)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # Timed region 2, each kernel's own time: the same K steps with HIP
    # events recorded on the launch stream around every launch.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        sw.swiglu_gateup_fwd(x, y)
        ev[k][1].record(stream)
        sw.swiglu_gateup_bwd(dy, x, dx)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    ms_per_step_with_events = (time.perf_counter() - t2) * 1e3 / K
    fwd_ms = [ev[k][0].elapsed_time(ev[k][1]) for k in range(K)]
    bwd_ms = [ev[k][1].elapsed_time(ev[k][2]) for k in range(K)]
    fwd_avg, bwd_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    log(f"[bench] step {ms_per_step:.4f} ms -> {value:.1f} GB/s ({ms_per_step_with_events:.4f} ms "
        f"with events); fwd {fwd_avg:.4f} ms, bwd {bwd_avg:.4f} ms")

    # The outputs of the timed step, kept for the oracle comparison in the
    # CPU-baseline leg (later legs overwrite y and dx).
    timed_outputs = None
    if not args.no_cpu_baseline:
        def stored(t, cols):
            a = t.reshape(w.rows, cols)
            if w.dtype == "bf16":
                return a.view(torch.int16).cpu().numpy().view(np.uint16)
            return a.cpu().numpy()
        timed_outputs = (stored(y, w.n), stored(dx, 2 * w.n))

    passes = {
        "fwd": {"ms_avg": round(fwd_avg, 5), "ms_median": round(float(np.median(fwd_ms)), 5),
                "ms_min": round(min(fwd_ms), 5), "ms_max": round(max(fwd_ms), 5),
                "GBps": round(fwd_bytes / fwd_avg / 1e6, 1), "bytes": fwd_bytes},
        "bwd": {"ms_avg": round(bwd_avg, 5), "ms_median": round(float(np.median(bwd_ms)), 5),
                "ms_min": round(min(bwd_ms), 5), "ms_max": round(max(bwd_ms), 5),
                "GBps": round(bwd_bytes / bwd_avg / 1e6, 1), "bytes": bwd_bytes},
        "fwd+bwd_kernels": {"ms_avg": round(fwd_avg + bwd_avg, 5),
                            "GBps": round(step_bytes / (fwd_avg + bwd_avg) / 1e6, 1)},
        "step_with_events": {"ms": round(ms_per_step_with_events, 5),
                             "GBps": round(step_bytes / ms_per_step_with_events / 1e6, 1),
                             "what": "the timed region of the per-kernel events (three per step)"},
    }

    if not args.no_extras:
        # In-place backward: each timed launch overwrites a fresh copy of x,
        # restored outside the timed events.
        x0 = x.detach().clone()
        ip_ms = []
        for k in range(max(5, K // 2) + 2):
            x.copy_(x0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sw.swiglu_gateup_bwd(dy, x, in_place=True)
            b.record(stream)
            b.synchronize()
            if k >= 2:
                ip_ms.append(a.elapsed_time(b))
        x.copy_(x0)
        del x0
        ip_avg = float(np.mean(ip_ms))
        passes["bwd_in_place"] = {"ms_avg": round(ip_avg, 5), "ms_min": round(min(ip_ms), 5),
                                  "GBps": round(bwd_bytes / ip_avg / 1e6, 1), "bytes": bwd_bytes}
        # A plain copy moving the backward's byte count (read half, write half)
        # as the empirical streaming ceiling, for context.
        nbytes = bwd_bytes // 2
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        cms = []
        for k in range(12):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            b.synchronize()
            if k >= 2:
                cms.append(a.elapsed_time(b))
        cavg = float(np.mean(cms))
        passes["copy_same_bytes"] = {"ms_avg": round(cavg, 5),
                                     "GBps": round(2 * nbytes / cavg / 1e6, 1),
                                     "bytes": 2 * nbytes, "kind": "torch copy_ (context)"}
        del src, dst
        log(f"[bench] bwd in_place {ip_avg:.4f} ms; copy {cavg:.4f} ms")
        # The same step through the autograd module (forward + loss-side
        # backward), and the two-tensor entry points on views of x.
        from swiglu_activation_amd.autograd import MegatronSwiGLU
        m = MegatronSwiGLU()
        xa = x.detach().requires_grad_(True)

        def ag_step():
            xa.grad = None
            m(xa).backward(dy)

        for _ in range(3):
            ag_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            ag_step()
        torch.cuda.synchronize()
        ag_ms = (time.perf_counter() - t0) * 1e3 / K
        passes["autograd_step"] = {"ms": round(ag_ms, 5), "GBps": round(step_bytes / ag_ms / 1e6, 1),
                                   "what": "MegatronSwiGLU forward + backward via autograd"}
        del xa
        gate, upv = x.reshape(w.rows, 2 * w.n)[:, :w.n], x.reshape(w.rows, 2 * w.n)[:, w.n:]
        dy2 = dy.reshape(w.rows, w.n)
        y2 = y.reshape(w.rows, w.n)
        dg2, du2 = dx.reshape(w.rows, 2 * w.n)[:, :w.n], dx.reshape(w.rows, 2 * w.n)[:, w.n:]
        tf, tb = pair_times(stream, lambda: sw.swiglu_silu_mul_fwd(gate, upv, y2),
                            lambda: sw.swiglu_silu_mul_bwd(dy2, gate, upv, dg2, du2), 10)
        passes["two_tensor_views"] = {"fwd_ms": round(tf, 5), "bwd_ms": round(tb, 5),
                                      "roofline_fwd": hbm_roofline("swiglu_silu_mul fwd", fwd_bytes, tf),
                                      "roofline_bwd": hbm_roofline("swiglu_silu_mul bwd", bwd_bytes, tb),
                                      "fwd_GBps": round(fwd_bytes / tf / 1e6, 1),
                                      "bwd_GBps": round(bwd_bytes / tb / 1e6, 1)}
        log(f"[bench] autograd step {ag_ms:.4f} ms; two-tensor fwd {tf:.4f} ms bwd {tb:.4f} ms")
        passes["bias_scale"] = bias_scale_leg(dev, stream, w, x, dy, y, dx)
        log(f"[bench] bias+scale fwd {passes['bias_scale']['fwd_ms']:.4f} ms, "
            f"bwd {passes['bias_scale']['bwd_ms']:.4f} ms")
        passes["other_workloads"], config_samples = configs_leg(
            dev, stream, [k for k in synth.WORKLOADS if k != w.name])
        log("[bench] other workloads: " + ", ".join(
            f"{k} fwd {v['fwd_GBps']:.0f} bwd {v['bwd_GBps']:.0f} GB/s"
            for k, v in passes["other_workloads"].items()))
        passes["fc1_swiglu"] = fc1_leg(dev, stream, w.rows)
        if (w.n * e) % 16 == 0 and w.rows <= 65535:
            passes["ceiling"] = ceiling_leg(dev, stream, w, x, dy, y, dx, fwd_avg, bwd_avg)
            cb = passes["ceiling"]["best"]
            log(f"[bench] ceiling: fwd mix best {cb['fwd']['GBps']:.0f} GB/s "
                f"({cb['fwd']['best_structure']}), bwd mix best {cb['bwd']['GBps']:.0f} GB/s "
                f"({cb['bwd']['best_structure']}); independent best fwd "
                f"{cb['fwd']['best_independent_GBps']:.0f}, bwd {cb['bwd']['best_independent_GBps']:.0f}")

    if args.calib:
        calib_copies(dev)

    achieved = bwd_bytes / (bwd_avg * 1e-3) / 1e9
    traffic = read_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.rows, "S": w.shape[0] if len(w.shape) == 3 else None,
                   "B": w.shape[1] if len(w.shape) == 3 else None, "n": w.n,
                   "x_shape": list(w.shape), "step": "forward + out-of-place backward",
                   "bytes_per_step": step_bytes},
        "pct_of_peak": round(100.0 * value / PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": "swiglu_bwd_kernel (out of place)",
                     "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": traffic},
        "passes": passes,
        "kernel_source_sha256_16": source_digest(),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle for about {args.cpu_seconds} s")
        out["cpu_baseline"] = cpu_baseline(w, x_h, dy_h, args.cpu_seconds, timed_outputs)
        if not args.no_extras:
            # the oracle against sampled rows of every other workload's timed outputs
            for name, smp in config_samples.items():
                wk = synth.WORKLOADS[name]
                passes["other_workloads"][name]["parity"] = oracle_parity_of_sample(wk.dtype, wk.n, smp)
            del config_samples
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
