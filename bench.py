#!/usr/bin/env python3
"""Benchmark: FP16-input / FP32-accumulate GEMM on one MI355X (gfx950).

One "step" is one call of the whole hot path, C = alpha*A@B + beta*C, on one
synthetic workload already resident in HBM.  The headline workload is the
2048^3 product (uniform[-1,1] inputs, alpha=1, beta=0); the 8192^3 roofline
shape and the other workloads are timed too and reported under "workloads"
in the same JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Timing: --settle-ms (default 100) of back-to-back launches of the same call
(the board ramps its clocks over the first ~25 ms of load after idle), then W
untimed warm-up steps, then exactly K steps bracketed by
torch.cuda.synchronize() on both sides (wall clock -> ms_per_step), with HIP
events recorded on the launch stream around the same region (-> the average
kernel duration used for the roofline); then, outside the timed region, the
pages' 5 runs x 20 launches ("timing": median of the runs' means and their
coefficient of variation).  FLOP = 2*M*N*K.  Each workload also reports "graph_us": the
per-launch time of the same call captured in a HIP graph and replayed, i.e.
the kernels' own time without the Python call between launches (which bounds
the eager rate of the smallest products).

For the 2048^3 headline the bench also measures the L2 fill and hit rates
per XCD with the diagnostics library's fill probe ("fill_rate").

The CPU baseline is the oracle (oracle/, plain C, FP64) timed on a bounded
sample of the headline workload: a block of whole rows of C, sized to about
--cpu-seconds of work on the host cores.  The same rows of the GPU result are
checked against it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (no sparsity): FP16 matrix cores and HBM3E.
PEAK_F16_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = ("FP16->FP32 GEMM TFLOP/s at 2048^3 (headline) and 8192^3; "
          "% of MI355X dense FP16 MFMA peak")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # The board ramps its clocks over the first ~1,000 back-to-back 2048^3
    # launches (~25 ms: 30.8 -> 24.0 us per launch); the default warm-up
    # covers that, so the timed steps see sustained throughput.
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="before the warm-up steps, launch the workload back to back for this long "
                        "(wall clock) so the board's clocks leave their idle state; 0 skips it")
    p.add_argument("--workload", default="square2048")
    p.add_argument("--config", type=int, default=None,
                   help="force this config-table entry for the headline workload (tile candidates)")
    p.add_argument("--candidates", action="store_true",
                   help="load the candidates build of the library (the product entries plus the "
                        "sweep-only tile shapes; python -m dense_mixed_precision_amd.build --candidates)")
    p.add_argument("--no-fill", dest="fill", action="store_false",
                   help="skip the L2 fill-rate probe")
    p.add_argument("--no-timeline", dest="timeline", action="store_false",
                   help="skip the per-workgroup timeline of the headline workload (timeline build)")
    p.add_argument("--no-breakdown", dest="breakdown", action="store_false",
                   help="skip the ragged workload's time breakdown")
    p.add_argument("--no-cold", dest="cold", action="store_false",
                   help="skip the cold-cache launches of the headline workload")
    p.add_argument("--no-others", action="store_true", help="time only the headline workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-power", dest="power", action="store_false",
                   help="skip the amd-smi power/clock sample under sustained 8192^3 load")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="after timing, run one plain device copy of this many MiB (a known-size "
                        "kernel for scaling the HBM byte counters of a rocprofv3 --pmc run)")
    return p.parse_args()


#: the product library as built in-tree
PRODUCT_LIB = os.path.join("dense_mixed_precision_amd", "libmpgemm.so")


def _elf_section(data: bytes, name: bytes):
    """(offset, size) of the named section of a 64-bit little-endian ELF file."""
    import struct

    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):
        return struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)

    strtab = header(shstrndx)[4]
    for i in range(shnum):
        name_off, _, _, _, off, size = header(i)
        end = data.index(b"\0", strtab + name_off)
        if data[strtab + name_off:end] == name:
            return off, size
    return None


def kernel_code_digest(lib: str | None = None):
    """Digest of the device code the product library carries (the code
    objects of every kernel in its .hip_fatbin section), or None if it is
    not built.  Counter readings are only reused while it matches: a change
    to host code alone (which table entry the factory picks) leaves it as it
    is, any change to a kernel or to the table's template arguments does
    not."""
    import hashlib

    path = lib or os.path.join(ROOT, PRODUCT_LIB)
    if not os.path.exists(path):
        return None
    with open(path, "rb") as f:
        data = f.read()
    sec = _elf_section(data, b".hip_fatbin")
    if sec is None:
        return None
    off, size = sec
    return hashlib.sha256(data[off:off + size]).hexdigest()[:16]


def measured_traffic(workload: str, kernel_ms: float):
    """Bytes per launch that leave the L2 caches for memory, from the committed
    rocprofv3 --pmc summary for this workload (FETCH_SIZE and WRITE_SIZE, each
    scaled by what it reads for a plain copy of known size), or None if there
    is none or the kernels changed since.  They count L2 misses, part of which
    the memory-side cache serves: an upper bound on DRAM bytes."""
    path = os.path.join(ROOT, "profiles", f"l2_miss_bytes_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    digest = kernel_code_digest()
    if digest is None or vals.get("kernel_code_digest") != digest:
        return None
    try:
        read_b = float(vals["l2_miss_read_bytes_per_launch"])
        write_b = float(vals["l2_miss_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    return {"bytes_per_launch": read_b + write_b, "read_bytes": read_b, "write_bytes": write_b,
            "GBps": round((read_b + write_b) / (kernel_ms * 1e-3) / 1e9, 1),
            "counts": "L2-to-memory requests (FETCH_SIZE, WRITE_SIZE), an upper bound on DRAM bytes",
            "source": os.path.relpath(path, ROOT)}


def graph_time_us(fn, reps, torch):
    """Per-launch time of `reps` calls captured in one HIP graph and replayed
    (best of three replays, HIP events on the replay stream): the kernels'
    own time without the Python call between launches.  `fn` launches on
    torch's current stream, which is the capture stream while capturing."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    best = float("inf")
    for _ in range(3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return best


def spread(ms):
    """Median, mean and coefficient of variation (stdev / mean) of per-launch
    times in ms, reported in microseconds."""
    import statistics

    mean = statistics.fmean(ms)
    cv = statistics.pstdev(ms) / mean if len(ms) > 1 and mean > 0 else 0.0
    return {"median_us": round(statistics.median(ms) * 1e3, 3), "mean_us": round(mean * 1e3, 3),
            "cv": round(cv, 4), "n": len(ms)}


def time_workload(w, steps, warmup, torch, mp, layout_a=0, layout_b=0, dtype=None, bias=False,
                  splitk=False, graph_reps=0, config=None, splits=0, runs=0, iters=20, sustained_ms=0.0,
                  settle_ms=0.0):
    """Time `steps` launches (after `warmup`) on resident inputs, then
    (`runs` > 0) `runs` more runs of `iters` launches each.  A column-
    major operand is stored transposed on the device and passed as the
    transposed view; `dtype` picks FP16 (default) or BF16 inputs; `bias`
    adds a per-column bias vector to the epilogue; `splitk` goes through the
    split-K entry point with `splits` pieces (0: the library's plan).
    `settle_ms` > 0: before the warm-up, launch back to back for that much
    wall time (the board ramps its clocks over the first ~25 ms of load)."""
    from dense_mixed_precision_amd.workloads import workload_inputs

    dev = torch.device("cuda:0")
    A, B, C = workload_inputs(w, dtype or torch.float16)
    Ad = A.t().contiguous().to(dev).t() if layout_a else A.to(dev)
    Bd = B.t().contiguous().to(dev).t() if layout_b else B.to(dev)
    Cd = C.to(dev) if C is not None else torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    cfg = mp.query_for(Ad, Bd, Cd, w.alpha, w.beta)
    if config is not None:
        cfg = dict(mp.mpgemm_config_info(config), grid=cfg["grid"])
    bias_d = torch.rand(w.N, device=dev) * 2 - 1 if bias else None
    ws = None
    if splitk:
        plan = mp.splitk_plan_for(Ad, Bd, Cd, splits)
        c = mp.mpgemm_config_info(plan["config_id"])
        tiles = -(-w.M // c["bm"]) * -(-w.N // c["bn"])
        cfg = dict(c, grid=cfg["grid"] if plan["splits"] == 1 else tiles * plan["splits"], splits=plan["splits"])
        ws = torch.empty(max(plan["workspace_bytes"] // 4, 1), dtype=torch.float32, device=dev)

    # The timed calls go through the raw C-ABI binding with the arguments
    # marshalled once (the tensor convenience wrapper re-checks strides and
    # dtypes on every call, ~10 us of Python that can leave a 25 us kernel's
    # queue empty): row-major FP16 without a bias calls mpgemm_f16f32 itself,
    # every other form mpgemm_gemm_ex.
    lda = w.M if layout_a else w.K
    ldb = w.K if layout_b else w.N
    handle = stream.cuda_stream
    a_ptr, b_ptr, c_ptr = Ad.data_ptr(), Bd.data_ptr(), Cd.data_ptr()
    bias_ptr = bias_d.data_ptr() if bias_d is not None else 0
    in_type = mp.MPGEMM_IN_BF16 if Ad.dtype == torch.bfloat16 else mp.MPGEMM_IN_F16
    alpha, beta = float(w.alpha), float(w.beta)
    plain = not splitk and not bias and not layout_a and not layout_b and in_type == mp.MPGEMM_IN_F16
    f16f32, gemm_ex, forced = mp.mpgemm_f16f32, mp.mpgemm_gemm_ex, mp.mpgemm_gemm_ex_with_config

    def step():
        if splitk:
            mp.gemm_splitk(Ad, Bd, Cd, w.alpha, w.beta, bias=bias_d, workspace=ws, stream=stream,
                           splits=splits)
            return
        if config is not None:
            rc = forced(config, in_type, layout_a, layout_b, w.M, w.N, w.K, a_ptr, lda, b_ptr, ldb, c_ptr,
                        w.N, alpha, beta, bias_ptr, handle)
        elif plain:
            rc = f16f32(w.M, w.N, w.K, a_ptr, lda, b_ptr, ldb, c_ptr, w.N, alpha, beta, handle)
        else:
            rc = gemm_ex(in_type, layout_a, layout_b, w.M, w.N, w.K, a_ptr, lda, b_ptr, ldb, c_ptr,
                         w.N, alpha, beta, bias_ptr, handle)
        if rc != mp.MPGEMM_OK:
            raise mp.MpgemmError(rc, "bench step")

    settle = None
    if settle_ms > 0:
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        n_settle = 0
        while (time.perf_counter() - s0) * 1e3 < settle_ms:
            for _ in range(64):
                step()
            n_settle += 64
            torch.cuda.synchronize()
        settle = {"launches": n_settle, "ms": round((time.perf_counter() - s0) * 1e3, 1)}
    for _ in range(warmup):
        step()
    # HIP events on the launch stream around the timed steps only: an event
    # recorded between steps costs about 2 us of queue time per 2048^3 step
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    kern_ms = ev0.elapsed_time(ev1) / steps
    out = {"A": A, "B": B, "C": C, "Cd": Cd, "cfg": cfg, "wall_ms": wall_ms, "kernel_ms": kern_ms,
           "settle": settle}
    if runs > 0:
        # the pages' method: `runs` runs of `iters` back-to-back launches,
        # each run's mean per launch; the median over runs and their spread
        run_ms = []
        for _ in range(runs):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            run_ms.append(e0.elapsed_time(e1) / iters)
        out["run_stats"] = dict(spread(run_ms), runs=runs, iters=iters)
    if sustained_ms > 0:
        # after `sustained_ms` of back-to-back launches (the board's clocks
        # settle within ~25 ms of load), the same 5 x 20 runs again
        n = max(1, int(sustained_ms * 1e3 / max(kern_ms * 1e3, 1.0)))
        for _ in range(n):
            step()
        run_ms = []
        for _ in range(max(runs, 5)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(iters):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            run_ms.append(e0.elapsed_time(e1) / iters)
        out["sustained"] = dict(spread(run_ms), after_launches=n, runs=max(runs, 5), iters=iters)
    if graph_reps > 0:
        # the same call on the current (capture) stream
        def step_current():
            if splitk:
                mp.gemm_splitk(Ad, Bd, Cd, w.alpha, w.beta, bias=bias_d, workspace=ws, splits=splits)
            else:
                mp.gemm(Ad, Bd, Cd, w.alpha, w.beta, bias=bias_d, config=config)

        out["graph_us"] = graph_time_us(step_current, graph_reps, torch)
    return out


def cold_timing(w, torch, mp, reps=20, scrub_mib=512):
    """Per-launch kernel time with cold caches: before each launch a
    `scrub_mib` MiB pass (twice the 256 MB memory-side cache) evicts the
    operands from the L2s and the memory-side cache; HIP events on the
    launch stream bracket the launch alone.  Two forms: the pass reads the
    buffer (the evicted lines are clean), or writes it (the product's reads
    then also push the pass's dirty lines out to HBM).  Medians over `reps`
    launches each (the timed steps run with warm caches, as the pages
    time)."""
    import statistics

    from dense_mixed_precision_amd.workloads import workload_inputs

    dev = torch.device("cuda:0")
    A, B, C = workload_inputs(w)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = C.to(dev) if C is not None else torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    scrub = torch.ones(scrub_mib * (1 << 18), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"reps": reps, "scrub_mib": scrub_mib,
           "note": "not the value: each launch after a pass over a 512 MiB buffer that evicts the L2s "
                   "and the memory-side cache; read: the pass reads it, write: the pass writes it"}
    for mode in ("read", "write", "read"):
        mp.gemm(Ad, Bd, Cd, w.alpha, w.beta)
        us = []
        for i in range(reps):
            if mode == "read":
                scrub.sum()
            else:
                scrub.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mp.gemm(Ad, Bd, Cd, w.alpha, w.beta)
            e1.record(stream)
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
        med = statistics.median(us)
        # the first read pass follows the buffer's initial write: keep the last
        out[mode] = {"median_us": round(med, 3), "min_us": round(min(us), 3), "max_us": round(max(us), 3),
                     "tflops": round(w.flop / (med * 1e-6) / 1e12, 2)}
    del scrub
    return out


def warmup_for(w, warmup):
    """Warm-up steps for a secondary workload: about 40 ms of GPU time (the
    clocks settle within ~25 ms of sustained load), at most `warmup`, at
    least 3 steps."""
    est_us = max(w.flop / 700e6, 5.0)  # rough time per launch in us at ~700 TFLOP/s
    return int(max(3, min(warmup, 40000.0 / est_us)))


def _smi_power():
    """Socket power (W) and mean graphics clock (MHz) from amd-smi, or None."""
    import re
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", "0"], capture_output=True,
                             text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    power = re.findall(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
    # the CLK line of each GFX_<n> section (one per XCD); other clock domains
    # (memory, video) have sections of their own
    clocks, section = [], ""
    for line in out.splitlines():
        m = re.match(r"^\s*([A-Z]+_?\d*):\s*$", line)
        if m:
            section = m.group(1)
            continue
        m = re.match(r"^\s*CLK:\s*([0-9.]+)\s*MHz", line)
        if m and section.startswith("GFX"):
            clocks.append(float(m.group(1)))
    if not power:
        return None
    return {"socket_w": float(power[0]),
            "gfx_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None,
            "gfx_sections": len(clocks)}


def sample_power(w, torch, mp, seconds=2.0):
    """Run workload `w` back to back for `seconds` and read socket power and
    the graphics clock in the middle of the run (outside any timed region):
    evidence for how far the board's power limit pulls the clock down under
    sustained matrix-core load."""
    import threading

    from dense_mixed_precision_amd.workloads import workload_inputs

    dev = torch.device("cuda:0")
    A, B, C = workload_inputs(w)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = C.to(dev) if C is not None else torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    idle = _smi_power()
    stop = time.perf_counter() + seconds
    count = [0]

    def loop():
        while time.perf_counter() < stop:
            for _ in range(10):
                mp.gemm(Ad, Bd, Cd, w.alpha, w.beta)
            torch.cuda.synchronize()
            count[0] += 10

    t0 = time.perf_counter()
    th = threading.Thread(target=loop)
    th.start()
    time.sleep(seconds * 0.6)
    busy = _smi_power()
    th.join()
    dt = time.perf_counter() - t0
    tflops = w.flop * count[0] / dt / 1e12
    out = {"workload": w.name, "idle": idle, "busy": busy,
           "tflops_during_sample": round(tflops, 1),
           "source": "amd-smi metric -p -c (SOCKET_POWER, graphics CLK of each XCD)"}
    if busy and busy.get("socket_w"):
        # work per joule of socket energy: what sets throughput at the power limit
        out["gflop_per_joule"] = round(tflops * 1e3 / busy["socket_w"], 1)
    return out


def mfma_ceiling(torch, mp, seconds=1.5):
    """Matrix-core-only throughput under sustained load: the library's
    throughput probe (independent matrix instructions, 128 accumulator
    registers per lane, no memory traffic) on one workgroup of 8 waves per
    compute unit, run back to back for `seconds` per case with socket power
    and the graphics clock read in the middle.  Cases: the 8192^3 workload's
    operand distribution (N(0,1) clipped to +-4) in FP16 on both
    instructions, constant FP16 operands, and the same random values in
    BF16.  What the board's power limit leaves for any FP16 kernel before
    operand traffic."""
    import threading

    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(77)
    rand = torch.randn(4096, generator=g).clamp_(-4.0, 4.0)
    cases = [("random_f16_16x16x32", mp.MPGEMM_IN_F16, 16, rand.to(torch.float16)),
             ("random_f16_32x32x16", mp.MPGEMM_IN_F16, 32, rand.to(torch.float16)),
             ("constant_f16_16x16x32", mp.MPGEMM_IN_F16, 16, torch.full((4096,), 1.0, dtype=torch.float16)),
             ("random_bf16_16x16x32", mp.MPGEMM_IN_BF16, 16, rand.to(torch.bfloat16))]
    wgs, iters = 256, 4000
    out = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    res = {}
    for name, in_type, shape, vals in cases:
        ops = vals.to(dev)
        per_round = 2 * 32 * 32 * 16 * 8 if shape == 32 else 2 * 16 * 16 * 32 * 32
        flop = wgs * 8 * iters * per_round

        def launch():
            rc = mp.mpgemm_probe_mfma_rate(in_type, shape, ops.data_ptr(), ops.numel(), iters, wgs,
                                           out.data_ptr(), out.numel(), torch.cuda.current_stream().cuda_stream)
            if rc != mp.MPGEMM_OK:
                raise mp.MpgemmError(rc, "mpgemm_probe_mfma_rate")

        for _ in range(20):
            launch()
        torch.cuda.synchronize()
        stop = time.perf_counter() + seconds
        count = [0]
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def loop():
            e0.record()
            while time.perf_counter() < stop:
                for _ in range(10):
                    launch()
                count[0] += 10
                torch.cuda.synchronize()
            e1.record()
            torch.cuda.synchronize()

        th = threading.Thread(target=loop)
        th.start()
        time.sleep(seconds * 0.6)
        busy = _smi_power()
        th.join()
        ms = e0.elapsed_time(e1)
        res[name] = {"tflops": round(flop * count[0] / (ms * 1e-3) / 1e12, 1), "launches": count[0],
                     "socket_w": busy and busy.get("socket_w"), "gfx_mhz_mean": busy and busy.get("gfx_mhz_mean")}
    res["source"] = ("mpgemm_probe_mfma_rate, 256 workgroups x 8 waves, 4000 rounds per launch; "
                     "amd-smi metric -p -c in the middle of each run")
    return res


def fill_rate(torch, mp):
    """L2 fill and hit rates per XCD from the diagnostics library's fill probe
    (256 workgroups of 8 waves, workgroup b on XCD b % 8; each XCD sweeps its
    own region of the buffer, every byte once per pass).  A 6 MiB region per
    XCD -- the footprint of a 2048^3 launch on one XCD, more than its 4 MiB
    L2 -- misses on every pass, so it measures the fill from the memory-side
    cache, which holds the whole 48 MiB buffer; a 2 MiB region stays in L2
    and measures hits.  Cases: the GEMM's copy form (16 bytes per lane into
    LDS) and 16- and 4-byte loads into registers at 1..16 requests in
    flight per wave; the copy form with every XCD reading the same region,
    and with each byte requested by 8 compute units of the XCD at once, as
    the 2048^3 kernel's workgroups sharing a panel do.  Per compute unit:
    the copy form with one workgroup per XCD (a lone compute unit's copy
    path) and the all-CU hit rate divided by 32.  Best of 3 timed launches
    after one untimed; GB/s per XCD (per CU) of unique bytes."""
    dev = torch.device("cuda:0")
    MiB = 1 << 20
    buf = torch.ones(48 * MiB // 4, dtype=torch.float32, device=dev)
    wgs = 256
    sink = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(wgs * 4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    names = {mp.MPGEMM_FILL_LDS16: "lds16", mp.MPGEMM_FILL_REG16: "reg16", mp.MPGEMM_FILL_REG4: "reg4"}
    ghz = {}

    def measure(mode, depth, footprint, shared=0, replicas=1, workgroups=wgs, key=None):
        passes = max(4, int(64 * 6 * MiB // footprint)) if workgroups == wgs else 16
        args = (mode, depth, buf.data_ptr(), buf.numel() * 4, footprint, shared, replicas, passes, workgroups,
                sink.data_ptr(), sink.numel(), clocks.data_ptr(), clocks.numel(), stream.cuda_stream)
        rc = mp.mpgemm_probe_fill(*args)
        if rc != mp.MPGEMM_OK:
            raise mp.MpgemmError(rc, "mpgemm_probe_fill")
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mp.mpgemm_probe_fill(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        if key is not None:
            c = clocks[:4 * workgroups].view(workgroups, 4).cpu().double()
            ghz[key] = round(float(((c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6)).median()) / 1e9, 3)
        return round(footprint * passes / best / 1e9, 1)

    out = {"per_xcd_GBps": {}, "unit": "GB/s per XCD (unique bytes)"}
    for mode in (mp.MPGEMM_FILL_LDS16, mp.MPGEMM_FILL_REG16, mp.MPGEMM_FILL_REG4):
        for depth in (1, 2, 4, 8, 16):
            out["per_xcd_GBps"][f"fill_6MiB_{names[mode]}_d{depth}"] = measure(mode, depth, 6 * MiB)
    out["per_xcd_GBps"]["fill_6MiB_lds16_d8_shared"] = measure(mp.MPGEMM_FILL_LDS16, 8, 6 * MiB, shared=1)
    out["per_xcd_GBps"]["fill_6MiB_lds16_d8_x8cu"] = measure(mp.MPGEMM_FILL_LDS16, 8, 6 * MiB, replicas=8)
    for depth in (2, 4, 8, 16):
        out["per_xcd_GBps"][f"hit_2MiB_lds16_d{depth}"] = measure(mp.MPGEMM_FILL_LDS16, depth, 2 * MiB)
    # one workgroup per XCD: what a single compute unit's copy path moves
    out["per_cu_GBps"] = {}
    for depth in (1, 2, 4, 8, 16):
        key = f"hit_2MiB_lds16_d{depth}_1cu"
        out["per_cu_GBps"][key] = measure(mp.MPGEMM_FILL_LDS16, depth, 2 * MiB, workgroups=8, key=key)
    for depth in (2, 8):
        key = f"hit_2MiB_lds16_d{depth}_32cu"
        out["per_cu_GBps"][key] = round(measure(mp.MPGEMM_FILL_LDS16, depth, 2 * MiB, key=key) / 32, 1)
    # a stream from HBM: 128 MiB per XCD (1 GiB in all, four times the
    # memory-side cache), each byte once per pass
    big = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    out["stream_GBps"] = {}
    for mode, depth in ((mp.MPGEMM_FILL_LDS16, 4), (mp.MPGEMM_FILL_LDS16, 8), (mp.MPGEMM_FILL_LDS16, 16),
                        (mp.MPGEMM_FILL_REG16, 8)):
        args = (mode, depth, big.data_ptr(), big.numel() * 4, 128 * MiB, 0, 1, 2, wgs, sink.data_ptr(),
                sink.numel(), 0, 0, stream.cuda_stream)
        rc = mp.mpgemm_probe_fill(*args)
        if rc != mp.MPGEMM_OK:
            raise mp.MpgemmError(rc, "mpgemm_probe_fill")
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            mp.mpgemm_probe_fill(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        out["stream_GBps"][f"stream_1GiB_{names[mode]}_d{depth}"] = round((1 << 30) * 2 / best / 1e9, 1)
    del big
    # the same in bytes per shader clock (each case's median workgroup clock)
    out["shader_clock_GHz"] = ghz
    out["per_cu_bytes_per_clk"] = {k: round(v / ghz[k], 1) for k, v in out["per_cu_GBps"].items()}
    vals = out["per_xcd_GBps"]
    out["best_fill_GBps"] = max(v for k, v in vals.items() if k.startswith("fill_6MiB_") and "_x8cu" not in k)
    out["best_hit_GBps"] = max(v for k, v in vals.items() if k.startswith("hit_"))
    out["best_per_cu_GBps"] = max(out["per_cu_GBps"].values())
    out["source"] = ("mpgemm_probe_fill (libmpgemm_probes.so), 256 workgroups x 8 waves (per_cu: 8 "
                     "workgroups, one per XCD), best of 3")
    del buf, sink
    return out


def ragged_breakdown(torch, mp, rounds=3, reps=50):
    """Where the ragged workload's time goes: graph-replayed per-launch time
    of the 1000x800x617 product (alpha 1.5, beta 0.5, lda 617) and of
    variants that each remove one of its features -- the C read (beta 0),
    the odd row stride of A (rows padded to 624 elements, 16-byte aligned),
    the K tail (K 616, a multiple of 8) -- beside the same product with one
    K tile (K 128), a single 64x64 workgroup with 5 and 1 K tiles, and the
    launch floor (a 16x16 product with K 0: the scale kernel alone).  The
    cases are timed in `rounds` interleaved rounds; best per case, in us.
    Inputs: the ragged workload's A, B and C (A copied into padded rows)."""
    from dense_mixed_precision_amd.workloads import WORKLOADS, workload_inputs

    dev = torch.device("cuda:0")
    w = WORKLOADS["ragged1000x800x617"]
    A, B, C = workload_inputs(w)
    a617 = A.to(dev)
    a624 = torch.zeros((w.M, 624), dtype=A.dtype, device=dev)
    a624[:, :w.K] = a617
    Bd = B.to(dev)
    C0 = C.to(dev)
    Cd = C0.clone()
    cases = {
        "workload": (w.M, w.N, 617, a617, 617, w.alpha, w.beta),
        "beta0": (w.M, w.N, 617, a617, 617, w.alpha, 0.0),
        "beta0_lda624": (w.M, w.N, 617, a624, 624, w.alpha, 0.0),
        "beta0_lda624_k616": (w.M, w.N, 616, a624, 624, w.alpha, 0.0),
        "beta0_lda624_k128": (w.M, w.N, 128, a624, 624, w.alpha, 0.0),
        "one_workgroup_k616": (64, 64, 616, a624, 624, w.alpha, 0.0),
        "one_workgroup_k128": (64, 64, 128, a624, 624, w.alpha, 0.0),
        "launch_floor_k0": (16, 16, 0, a624, 624, w.alpha, 0.0),
    }
    best = {k: float("inf") for k in cases}
    for _ in range(rounds):
        for name, (M, N, K, a, lda, alpha, beta) in cases.items():
            def step(M=M, N=N, K=K, a=a, lda=lda, alpha=alpha, beta=beta):
                # torch's current stream: the capture stream while a graph is captured
                rc = mp.mpgemm_f16f32(M, N, K, a.data_ptr(), lda, Bd.data_ptr(), w.N, Cd.data_ptr(), w.N,
                                      alpha, beta, torch.cuda.current_stream(dev).cuda_stream)
                if rc != mp.MPGEMM_OK:
                    raise mp.MpgemmError(rc, f"ragged breakdown {name}")
            Cd.copy_(C0)
            for _ in range(300):
                step()
            torch.cuda.synchronize()
            best[name] = min(best[name], graph_time_us(step, reps, torch))
    if min(best.values()) < 0.5:
        # no kernel takes less than a launch: the graph captured nothing
        raise RuntimeError(f"ragged breakdown timed an empty graph: {best}")
    t = {k: round(v, 3) for k, v in best.items()}
    return {
        "us": t,
        "c_read_us": round(t["workload"] - t["beta0"], 3),
        "odd_row_stride_us": round(t["beta0"] - t["beta0_lda624"], 3),
        "k_tail_us": round(t["beta0_lda624"] - t["beta0_lda624_k616"], 3),
        "per_k_tile_us": round((t["beta0_lda624_k616"] - t["beta0_lda624_k128"]) / 4, 3),
        "per_k_tile_one_workgroup_us": round((t["one_workgroup_k616"] - t["one_workgroup_k128"]) / 4, 3),
        "launch_floor_us": t["launch_floor_k0"],
        "note": "graph-replayed per-launch times, best of interleaved rounds; K tiles are 128 deep (5 for "
                "K 616/617, 1 for K 128)",
    }


def timeline_summary(rec, nwg):
    """Summary of one launch's timeline records (uint64 array of shape
    [>= nwg, 48], layout in include/mpgemm_timeline.h).  Each workgroup's
    shader clock is its shader-clock span over its 100 MHz-clock span; its
    intervals are converted with its own clock.  Medians over the
    workgroups of: the start skew, the wait from the start to the first
    published K tile, the interval between consecutive publishes (per tile
    index, for the tiles recorded), the time from the last recorded publish
    to the end of the K loop, and the epilogue; plus each XCD's median end.
    Times in microseconds."""
    import numpy as np

    r = np.asarray(rec[:nwg], dtype=np.uint64).astype(np.int64)
    clk = (r[:, 45] - r[:, 1]) / ((r[:, 46] - r[:, 0]) / 100e6)

    def us(a, b):
        return (r[:, b] - r[:, a]) / clk * 1e6

    def med(x):
        return round(float(np.median(x)), 3)

    t0 = r[:, 0].min()
    start = (r[:, 0] - t0) / 100.0
    end = (r[:, 46] - t0) / 100.0
    ntiles = int(r[0, 43])
    nrec = min(ntiles, 41)
    intervals = [med(us(1 + t, 2 + t)) for t in range(1, nrec)]
    last = 1 + nrec
    xcd = (r[:, 47] >> 32) & 0xF
    return {
        "workgroups": int(nwg),
        "k_tiles": ntiles,
        "shader_clock_GHz": round(float(np.median(clk)) / 1e9, 3),
        "start_skew_us": {"median": med(start), "max": round(float(start.max()), 3)},
        "first_tile_us": med(us(1, 2)),
        "tile_interval_us": intervals,
        "steady_tile_interval_us": med(np.array(intervals[2:] or intervals or [0.0])),
        "last_recorded_tile_to_loop_end_us": med(us(last, 44)),
        "tiles_after_last_recorded": ntiles - nrec,
        "epilogue_us": med(us(44, 45)),
        "workgroup_us": med(us(1, 45)),
        "launch_span_us": round(float(end.max()), 3),
        "xcd_end_us": {int(x): med(end[xcd == x]) for x in sorted(set(xcd.tolist()))},
    }


def timeline(w, torch, mp, warm=200, launches=3):
    """Per-workgroup timeline of the factory's kernel for `w` from the
    timeline build (libmpgemm_timeline.so, loaded beside the product): after
    `warm` back-to-back launches the records of the last one are read, three
    times; the summary of the median launch (by span) is returned.  None
    when the factory picks a kernel other than the pipelined one."""
    import numpy as np

    from dense_mixed_precision_amd.workloads import workload_inputs

    dev = torch.device("cuda:0")
    A, B, C = workload_inputs(w)
    Ad, Bd = A.to(dev), B.to(dev)
    Cd = C.to(dev) if C is not None else torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    cfg = mp.query_for(Ad, Bd, Cd, w.alpha, w.beta)
    if cfg["kind_name"] != "pipe":
        return None
    lib = mp.load_timeline()
    nwg = min(int(cfg["grid"]), 4096)
    handle = torch.cuda.current_stream(dev).cuda_stream
    if lib.mpgemm_timeline_clear() != mp.MPGEMM_OK:
        raise mp.MpgemmError(mp.MPGEMM_ELAUNCH, "mpgemm_timeline_clear")
    rec = np.zeros((nwg, mp.TIMELINE_SLOTS), dtype=np.uint64)
    runs = []
    for _ in range(launches):
        if C is not None:
            Cd.copy_(C.to(dev))
        for _ in range(warm):
            rc = lib.mpgemm_f16f32(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N, Cd.data_ptr(), w.N,
                                   float(w.alpha), float(w.beta), handle)
            if rc != mp.MPGEMM_OK:
                raise mp.MpgemmError(rc, "timeline build launch")
        rc = lib.mpgemm_timeline_read(rec.ctypes.data, rec.size)
        if rc != mp.MPGEMM_OK:
            raise mp.MpgemmError(rc, "mpgemm_timeline_read")
        runs.append(timeline_summary(rec, nwg))
    runs.sort(key=lambda d: d["launch_span_us"])
    out = runs[len(runs) // 2]
    out["kernel"] = {k: cfg[k] for k in ("id", "bm", "bn", "bk", "stages", "mfma_m", "k_order", "grid")}
    out["source"] = ("libmpgemm_timeline.so (the product source with -DMPGEMM_TIMELINE): thread 0 of each "
                     f"workgroup stamps the shader clock; last of {warm} back-to-back launches, median of "
                     f"{launches}")
    return out


def copy_bound(w, cfg, tl, fill, kernel_ms):
    """The launch time this tiling allows when every compute unit's copies
    into LDS run at the best rate the fill probe measured for all compute
    units copying at once (bytes per shader clock), at the shader clock the
    timeline measured under this load: each workgroup copies (BM + BN) * K * 2
    bytes, plus the first-tile wait and the epilogue the timeline measured
    (they do not overlap the loop).  A bound for this decomposition, not for
    the product: another tiling moves other bytes."""
    per_cu = fill["per_cu_bytes_per_clk"]
    rate = max(v for k, v in per_cu.items() if k.endswith("_32cu"))
    ghz = tl["shader_clock_GHz"]
    copy_bytes = (cfg["bm"] + cfg["bn"]) * w.K * 2
    loop_us = copy_bytes / rate / (ghz * 1e3)
    # the first tile's copies are part of the first-tile wait
    loop_us *= (tl["k_tiles"] - 1) / tl["k_tiles"]
    bound_us = loop_us + tl["first_tile_us"] + tl["epilogue_us"]
    return {"copy_bytes_per_workgroup": copy_bytes, "copy_bytes_per_clk": rate, "shader_clock_GHz": ghz,
            "loop_us": round(loop_us, 3), "first_tile_us": tl["first_tile_us"], "epilogue_us": tl["epilogue_us"],
            "bound_us": round(bound_us, 3), "bound_tflops": round(w.flop / (bound_us * 1e-6) / 1e12, 1),
            "kernel_us": round(kernel_ms * 1e3, 3), "frac_of_bound": round(bound_us / (kernel_ms * 1e3), 3)}


def roofline_entry(w, kernel_ms):
    """MFMA bound for the compute-heavy shapes, HBM bound where the
    arithmetic intensity (FLOP per algorithmic byte) is below the ridge."""
    ai = w.flop / w.algorithmic_bytes
    ridge = PEAK_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        achieved = w.flop / (kernel_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": None}
    achieved = w.algorithmic_bytes / (kernel_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}


def with_traffic(roof, traffic):
    """`roof` with its traffic entry: the measured L2-miss bytes per launch
    (or None) and their detail."""
    roof = dict(roof)
    roof["traffic"] = traffic["bytes_per_launch"] if traffic else None
    roof["traffic_detail"] = traffic
    return roof


def cpu_baseline(w, res, seconds):
    """The oracle, as it stands, on whole rows of C of the headline workload."""
    import numpy as np

    import oracle
    from dense_mixed_precision_amd.workloads import bits

    Ab, Bb = bits(res["A"]), bits(res["B"])
    Cn = None if res["C"] is None else res["C"].numpy()
    got = res["Cd"].cpu().numpy() if w.beta == 0 else None

    def run_rows(r0, r1):
        a = np.ascontiguousarray(Ab[r0:r1])
        c = None if Cn is None else np.ascontiguousarray(Cn[r0:r1])
        t = time.perf_counter()
        ref, absdot = oracle.gemm(a, Bb, c, w.alpha, w.beta)
        return time.perf_counter() - t, ref, absdot

    # Whole rows, in blocks sized from the previous block's rate, until about
    # `seconds` of oracle time or the whole matrix.
    r0 = 0
    refs, absd = [], []
    dt = 0.0
    block = max(1, min(w.M, 8))
    while r0 < w.M and dt < seconds:
        t_block, ref_b, abs_b = run_rows(r0, min(w.M, r0 + block))
        refs.append(ref_b)
        absd.append(abs_b)
        dt += t_block
        r0 = min(w.M, r0 + block)
        per_row = t_block / ref_b.shape[0]
        block = int(max(1, min(w.M - r0, (seconds - dt) / max(per_row, 1e-9))))
    rows = r0
    ref, absdot = np.concatenate(refs), np.concatenate(absd)
    r0 = 0
    flop = 2.0 * rows * w.N * w.K
    out = {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of {w.M} ({rows} rows x {w.N} cols x K={w.K}) "
                     f"of {w.name}; {dt:.1f} s of oracle time",
           "seconds": round(dt, 2)}
    out["cpu_model"] = cpu_model()
    if got is not None:
        ok = oracle.tolerance_ok(got[r0:r0 + rows], ref, absdot)
        err = np.abs(got[r0:r0 + rows] - ref) / (oracle.TOL_REL * absdot + oracle.TOL_ABS)
        out["gpu_rows_match"] = bool(ok.all())
        out["gpu_rows_worst_err_over_tol"] = float(err.max())
        # the error against the worst case of an FP32 running sum (at most 1
        # for FP32 accumulation; an FP16 running sum exceeds it)
        epi = oracle.epilogue_abs(w.beta, None if Cn is None else Cn[r0:r0 + rows])
        out["gpu_rows_accumulation_ratio"] = oracle.accumulation_ratio(got[r0:r0 + rows], ref, absdot, w.K,
                                                                       w.alpha, epilogue_abs=epi)
    return out


def cpu_model() -> str:
    """The host CPU's model name (first "model name" of /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this GEMM path has "
              "no multi-GPU mode. Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    import dense_mixed_precision_amd as mp
    from dense_mixed_precision_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mp.load(mp.CANDIDATES_PATH if args.candidates else None)
    if args.config is not None and not 0 <= args.config < mp.mpgemm_num_configs():
        print(f"config {args.config} is not in {mp.lib_path()} ({mp.mpgemm_num_configs()} entries; the "
              "sweep-only shapes need --candidates)", file=sys.stderr)
        sys.exit(2)
    head = WORKLOADS[args.workload]
    print(f"# timing {head.name} ({args.warmup} warm-up + {args.steps} steps)", file=sys.stderr, flush=True)
    res = time_workload(head, args.steps, args.warmup, torch, mp, graph_reps=20, config=args.config, runs=5,
                        iters=20, sustained_ms=50.0, settle_ms=args.settle_ms)
    value = head.flop / (res["wall_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": head.name, "M": head.M, "N": head.N, "K": head.K,
                   "alpha": head.alpha, "beta": head.beta, "inputs": head.dist,
                   "accumulate": "f32", "output": "f32", "layout": "row-major A, B, C",
                   "kernel": {k: res["cfg"][k] for k in ("id", "kind_name", "bm", "bn", "bk", "wave_m",
                                                        "wave_n", "vec_a", "vec_b", "grid")},
                   "pct_of_peak": round(100 * value / PEAK_F16_TFLOPS, 2),
                   "peak_tflops": PEAK_F16_TFLOPS},
        "roofline": roofline_entry(head, res["kernel_ms"]),
    }
    line["roofline"]["kernel_ms"] = round(res["kernel_ms"], 5)
    if res["settle"]:
        line["settle"] = dict(res["settle"], note="before the warm-up steps, back-to-back launches of the same "
                              "call for --settle-ms of wall time: the board ramps its clocks over the first "
                              "~25 ms of load (2048^3: 30.8 -> 24 us per launch), so the timed steps see "
                              "the sustained clock; the other workloads get the same settle")
    traffic = measured_traffic(head.name, res["kernel_ms"])
    line["roofline"]["traffic"] = traffic["bytes_per_launch"] if traffic else None
    line["roofline"]["traffic_detail"] = traffic
    sus = res["sustained"]
    line["sustained"] = {"median_us": sus["median_us"], "cv": sus["cv"],
                         "tflops": round(head.flop / (sus["median_us"] * 1e-6) / 1e12, 2),
                         "after_launches": sus["after_launches"],
                         "note": "not the value: 5 runs of 20 launches after ~50 ms of back-to-back launches "
                                 "(the clocks settle under sustained load), after the timed steps"}
    line["timing"] = {"runs_5x20": res["run_stats"],
                      "note": "per-launch kernel time from HIP events on the launch stream over 5 runs of 20 "
                              "back-to-back launches after the timed steps: median of the runs' means, CV "
                              "across runs (the pages' medians of 5 x 20)"}
    line["graph_us"] = round(res["graph_us"], 3)
    if args.cold and args.config is None:
        print("# cold-cache launches", file=sys.stderr, flush=True)
        line["cold"] = cold_timing(head, torch, mp)
    if args.timeline and args.config is None:
        print("# per-workgroup timeline (timeline build)", file=sys.stderr, flush=True)
        line["timeline"] = timeline(head, torch, mp, warm=max(5, min(200, int(2e13 / head.flop))))
    if args.breakdown and (head.name == "ragged1000x800x617" or not args.no_others) and args.config is None:
        print("# ragged breakdown", file=sys.stderr, flush=True)
        line["ragged_breakdown"] = ragged_breakdown(torch, mp)
    if args.fill and head.name == "square2048" and args.config is None:
        print("# L2 fill-rate probe", file=sys.stderr, flush=True)
        line["fill_rate"] = fill_rate(torch, mp)
        if line.get("timeline"):
            line["copy_bound"] = copy_bound(head, res["cfg"], line["timeline"], line["fill_rate"],
                                            res["kernel_ms"])
    others = {}
    if not args.no_others:
        for name, w in WORKLOADS.items():
            if name == head.name:
                continue
            steps = max(5, min(args.steps, 20 if w.flop > 1e12 else args.steps))
            print(f"# timing {name} ({steps} steps)", file=sys.stderr, flush=True)
            r = time_workload(w, steps, warmup_for(w, args.warmup), torch, mp,
                              graph_reps=5 if w.flop > 1e12 else 20, settle_ms=args.settle_ms)
            others[name] = {"tflops": round(w.flop / (r["kernel_ms"] * 1e-3) / 1e12, 2),
                            "kernel_ms": round(r["kernel_ms"], 5), "wall_ms": round(r["wall_ms"], 5),
                            "graph_us": round(r["graph_us"], 3),
                            "pct_of_peak": round(100 * w.flop / (r["kernel_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
                            "roofline": with_traffic(roofline_entry(w, r["kernel_ms"]),
                                                     measured_traffic(name, r["kernel_ms"])),
                            "kernel": {k: r["cfg"][k] for k in ("id", "kind_name", "bm", "bn", "vec_a", "vec_b",
                                                                "grid")}}
            del r
            torch.cuda.empty_cache()
        # the column-major operand modes, BF16 inputs and the bias epilogue
        # on the two headline shapes
        variants = [(0, 1, None, False, "Bcol"), (1, 1, None, False, "AcolBcol"),
                    (0, 0, torch.bfloat16, False, "bf16"), (0, 1, torch.bfloat16, False, "bf16_Bcol"),
                    (0, 0, None, True, "bias")]
        for base in ("square2048", "square8192"):
            w = WORKLOADS[base]
            for la, lb, dt, with_bias, tag in variants:
                name = f"{base}_{tag}"
                steps = max(5, min(args.steps, 20 if w.flop > 1e12 else args.steps))
                print(f"# timing {name} ({steps} steps)", file=sys.stderr, flush=True)
                r = time_workload(w, steps, warmup_for(w, args.warmup), torch, mp, la, lb, dt, with_bias,
                                  graph_reps=5 if w.flop > 1e12 else 20, settle_ms=args.settle_ms)
                others[name] = {"tflops": round(w.flop / (r["kernel_ms"] * 1e-3) / 1e12, 2),
                                "kernel_ms": round(r["kernel_ms"], 5), "wall_ms": round(r["wall_ms"], 5),
                                "graph_us": round(r["graph_us"], 3),
                                "layout": {"A": "col" if la else "row", "B": "col" if lb else "row"},
                                "inputs": "bf16" if dt is not None else "f16", "bias": with_bias,
                                "pct_of_peak": round(100 * w.flop / (r["kernel_ms"] * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 2),
                                "roofline": roofline_entry(w, r["kernel_ms"]),
                                "kernel": {k: r["cfg"][k] for k in ("id", "bm", "bn", "bk", "vec_a", "vec_b", "grid")}}
                del r
                torch.cuda.empty_cache()
        # the pages' skinny case on the tiled kernel split 8 ways over K, beside
        # the library's choice above (the narrow kernel)
        skinny = WORKLOADS["skinny4096x16x4096"]
        for tag, sk in (("_splitk8", 8),):
            name = skinny.name + tag
            print(f"# timing {name} ({args.steps} steps)", file=sys.stderr, flush=True)
            r = time_workload(skinny, args.steps, warmup_for(skinny, args.warmup), torch, mp, splitk=True,
                              graph_reps=20, splits=sk, settle_ms=args.settle_ms)
            others[name] = {"tflops": round(skinny.flop / (r["kernel_ms"] * 1e-3) / 1e12, 2),
                            "kernel_ms": round(r["kernel_ms"], 5), "wall_ms": round(r["wall_ms"], 5),
                            "graph_us": round(r["graph_us"], 3),
                            "roofline": roofline_entry(skinny, r["kernel_ms"]),
                            "splits": r["cfg"].get("splits", 1),
                            "kernel": {k: r["cfg"][k] for k in ("id", "kind_name", "bm", "bn", "bk", "grid")}}
            del r
            torch.cuda.empty_cache()
        line["workloads"] = others
    if args.power:
        line["power"] = sample_power(WORKLOADS["square8192"], torch, mp)
        print("# matrix-core ceiling (throughput probe under sustained load)", file=sys.stderr, flush=True)
        line["mfma_ceiling"] = mfma_ceiling(torch, mp)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(head, res, args.cpu_seconds)
    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb * 1024 * 1024 // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n * 4
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
