#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X: TFLOP/s and fraction of the MFMA roofline.

A step is one attention forward (the whole fused kernel) over one batch of
synthetic inputs already resident in HBM.  Default workload: B=1, H=16,
N=16384, d=128, bf16 (the long-sequence headline shape); the N=2048 fp32
shape (B=4, H=8, d=64, Q and K x4) is timed beside it as "secondary".

Prints ONE JSON line on stdout; progress goes to stderr.

Modes:
  python bench.py [--steps K] [--warmup W] [--config 5] [--secondary 3]
  python bench.py --profile-pass --config C     (a few launches plus a plain
      device copy of known size, for rocprofv3 counter runs)
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --config C
      (turns two rocprofv3 --pmc outputs into profiles/traffic.json)
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense matrix-core peaks (TFLOP/s) and HBM bandwidth (GB/s).
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3, "f64": 78.6}
HBM_PEAK_GBS = 8000.0
# The fp32 path's products run on the int8 and bf16 matrix cores from exact
# splits of the fp32 values.  Per 16 queries x 16 keys x 64 columns (65536
# counted flop) it issues 19 v_mfma_i32_16x16x64_i8 and 12
# v_mfma_f32_16x16x32_bf16, 16 cycles each: 132 counted flop per cycle per
# SIMD, 324.7 TFLOP/s over 1024 SIMDs at 2.4 GHz (the same at d = 128).
F32_ENGINE_PEAK_TFLOPS = 65536 / ((19 + 12) * 16) * 1024 * 2.4e9 / 1e12
# What each attention path computes in (the data type alone does not say it).
ARITH = {
    "bf16": "bf16 matrix products with fp32 accumulation, fp32 softmax",
    "f32": "int8 matrix products of exact int8 slices of the fp32 Q and K rows (int32 accumulation, "
           "fp64 combination); bf16 matrix products of exact three-piece bf16 splits of P and V "
           "(fp32 accumulation); fp64 running max and denominator, fp32 exp2",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 512 * 1024 * 1024  # calibration copy for the HBM byte counters


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# The sources each operation's kernels and launch code are built from.
OP_SOURCES = {
    "attn": ("common.hpp", "api_util.hpp", "attn_bf16.hpp", "attn_bf16_solo.hpp", "attn_f32.hpp", "hfa_api.hip"),
    "softmax": ("common.hpp", "hbm_io.hpp", "api_util.hpp", "softmax_rows.hpp", "softmax_api.hip"),
    "rmsnorm": ("common.hpp", "hbm_io.hpp", "api_util.hpp", "rmsnorm.hpp", "rmsnorm_api.hip"),
}


def kernel_source_digest(op: str = "attn") -> str:
    """Digest of one operation's HIP sources: counter figures are only valid for the kernel they were taken on.

    Line comments and whitespace are dropped first, so editing prose does not void figures
    taken on the same code."""
    h = hashlib.sha256()
    for name in sorted(OP_SOURCES[op]):
        with open(os.path.join(ROOT, "fa2_fwd_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        code = "".join(re.sub(r"//.*", "", line).strip() for line in text.splitlines())
        h.update(name.encode())
        h.update(re.sub(r"\s+", "", code).encode())
    return h.hexdigest()[:16]


def kernel_key(w) -> str:
    return f"attn_fwd_{w.dtype}_d{w.d}"


def algorithmic_bytes(w) -> int:
    """Q, K, V read once and O written once (elt bytes each) plus LSE (fp32)."""
    elt = 4 if w.dtype == "f32" else 2
    return 4 * w.B * w.H * w.N * w.d * elt + 4 * w.B * w.H * w.N


def load_traffic(w):
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    entry = table.get(kernel_key(w) + f"_N{w.N}")
    if not entry or entry.get("src_digest") != kernel_source_digest():
        return None
    return entry


# Seconds of untimed launches after the W warm-up steps, so that the shader
# clock has ramped before timing: a short kernel (0.27 ms at N=2048 fp32) times
# ~20 % slower after 10 launches than after 0.5 s of them.
CLOCK_RAMP_S = 0.5


def warm_up(launch, warmup: int, ramp_s: float) -> None:
    """W launches, then more of the same until ramp_s seconds have passed."""
    import torch

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < ramp_s:
        for _ in range(8):
            launch()
        torch.cuda.synchronize()


def attn_workspace(w, dev):
    """The workspace the library asks for on this workload (fp32 shapes whose key tiles
    are shared by enough workgroups: K and V formatted once per call; bf16: a key
    split), allocated once outside the timed region, or None."""
    import torch

    import fa2_fwd_amd as hfa

    code = hfa.HFA_F32 if w.dtype == "f32" else hfa.HFA_BF16
    need = hfa.hfa_attn_fwd_workspace_size(code, w.B, w.H, w.N, w.d, 0)
    return torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None


def time_gpu(w, steps: int, warmup: int, ramp_s: float = CLOCK_RAMP_S):
    import torch

    import fa2_fwd_amd as hfa
    from fa2_fwd_amd import workloads as W

    dev = torch.device("cuda:0")
    log(f"[bench] {w.describe()}: generating inputs")
    q, k, v = (t.to(dev) for t in W.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws = attn_workspace(w, dev)
    warm_up(lambda: hfa.attn_fwd(q, k, v, w.scale, out=o, lse=lse, stream=stream, workspace=ws), warmup, ramp_s)
    # One event before each launch and one after the last, all on the launch
    # stream: their span is the timed region, their gaps the per-launch times.
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        events[i].record(stream)
        hfa.attn_fwd(q, k, v, w.scale, out=o, lse=lse, stream=stream, workspace=ws)
    events[steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = events[0].elapsed_time(events[steps]) / steps
    per_launch = sorted(events[i].elapsed_time(events[i + 1]) for i in range(steps))
    tflops = w.flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    log(f"[bench] {w.describe()}: {ms:.4f} ms/launch, {tflops:.1f} TFLOP/s, {100 * tflops / peak:.1f}% of "
        f"{w.dtype} MFMA peak (wall {wall:.3f} s for {steps} steps)")
    traffic = load_traffic(w)
    roofline = {
        "bound": "mfma",
        "achieved": round(tflops, 3),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(tflops / peak, 4),
        "traffic": None if traffic is None else int(traffic["hbm_bytes_per_launch"]),
        "algorithmic_bytes": algorithmic_bytes(w),
        # HBM rates over the measured step: counted traffic (when taken on these sources) and
        # the algorithmic Q, K, V, O and LSE bytes
        "traffic_gbs": None if traffic is None else round(traffic["hbm_bytes_per_launch"] / (ms * 1e6), 1),
        "algorithmic_gbs": round(algorithmic_bytes(w) / (ms * 1e6), 1),
        "kernel": kernel_key(w),
    }
    if w.dtype == "f32":
        # The fp32 path issues int8 and bf16 matrix-core instructions, not fp32 ones: its
        # roofline is the ceiling of those instructions; the fp32 MFMA peak stays as context
        # (what fp32 matrix cores would allow for the same counted work).
        roofline["peak"] = round(F32_ENGINE_PEAK_TFLOPS, 1)
        roofline["frac"] = round(tflops / F32_ENGINE_PEAK_TFLOPS, 4)
        roofline["peak_basis"] = ("ceiling of the instructions issued: 19 v_mfma_i32_16x16x64_i8 + 12 "
                                  "v_mfma_f32_16x16x32_bf16 (16 cycles each) per 65536 counted flop")
        roofline["fp32_peak"] = peak
        roofline["fp32_frac"] = round(tflops / peak, 4)
    return {"ms": ms, "tflops": tflops, "wall_s": wall, "roofline": roofline,
            "ms_median": per_launch[len(per_launch) // 2], "ms_min": per_launch[0]}


def graph_time(w, count: int, reps: int):
    """Per-launch time when `count` launches are replayed from one captured graph."""
    import torch

    import fa2_fwd_amd as hfa
    from fa2_fwd_amd import workloads as W

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.workload_inputs(w))
    stream = torch.cuda.current_stream(dev)
    with hfa.AttnGraph(q, k, v, w.scale, count=count) as g:
        g.launch(stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.launch(stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * count)




def softmax_key(sw) -> str:
    return f"softmax_rows_f32_{sw.rows}x{sw.cols}"


def rmsnorm_key(rw) -> str:
    return f"rmsnorm_{rw.dtype}_{rw.rows}x{rw.cols}" + ("_res" if rw.residual else "")


def _softmax_launcher(sw):
    import torch

    import fa2_fwd_amd as hfa

    x = sw.inputs().cuda()
    y = torch.empty_like(x)
    return lambda stream: hfa.softmax_rows(x, out=y, stream=stream)


def _rmsnorm_launcher(rw):
    import torch

    import fa2_fwd_amd as hfa

    x, r, w = (None if t is None else t.cuda() for t in rw.inputs())
    y = torch.empty_like(x)
    s = torch.empty_like(x) if r is not None else None
    return lambda stream: hfa.rmsnorm(x, w, rw.eps, residual=r, out=y, residual_out=s, stream=stream)


def _softmax_oracle_rows(sw):
    import oracle

    x = sw.inputs().numpy()
    return lambda rows, threads: oracle.softmax_rows(x, rows=rows, threads=threads), "fp64 definition"


def _rmsnorm_oracle_rows(rw):
    import numpy as np
    import torch

    import oracle

    def host(t):
        if t is None:
            return None
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    x, r, w = (host(t) for t in rw.inputs())
    return (lambda rows, threads: oracle.rmsnorm(x, w, rw.eps, residual=r, rows=rows, threads=threads),
            "fp32 residual sum, fp64 normalisation")


# The HBM-bound operations timed beside the attention forward: their workloads,
# the marker of their kernels' names in a trace, and how to launch and check them.
HBM_OPS = {
    "softmax": dict(configs="SOFTMAX_CONFIGS", marker="softmax_rows", key=softmax_key,
                    launcher=_softmax_launcher, oracle_rows=_softmax_oracle_rows, json_key="softmax_rows"),
    "rmsnorm": dict(configs="RMSNORM_CONFIGS", marker="rmsnorm_kernel", key=rmsnorm_key,
                    launcher=_rmsnorm_launcher, oracle_rows=_rmsnorm_oracle_rows, json_key="rmsnorm"),
}


def hbm_configs(op: str):
    from fa2_fwd_amd import workloads as W

    return getattr(W, HBM_OPS[op]["configs"])


def load_op_traffic(op: str, wl):
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f).get(HBM_OPS[op]["key"](wl))
    except (OSError, ValueError):
        return None
    if not entry or entry.get("src_digest") != kernel_source_digest(op):
        return None
    return entry


def time_hbm_op(op: str, wl, steps: int, warmup: int):
    """One HBM-bound operation on inputs resident in HBM: ms per launch and algorithmic GB/s."""
    import torch

    launch = HBM_OPS[op]["launcher"](wl)
    stream = torch.cuda.current_stream()
    warm_up(lambda: launch(stream), warmup, CLOCK_RAMP_S)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        events[i].record(stream)
        launch(stream)
    events[steps].record(stream)
    torch.cuda.synchronize()
    ms = events[0].elapsed_time(events[steps]) / steps
    per = sorted(events[i].elapsed_time(events[i + 1]) for i in range(steps))
    gbs = wl.algorithmic_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] {wl.describe()}: {ms:.4f} ms/launch, {gbs:.0f} GB/s of algorithmic bytes, "
        f"{100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak")
    traffic = load_op_traffic(op, wl)
    return {
        "workload": wl.describe(),
        "ms_per_step": round(ms, 5),
        "ms_median": round(per[len(per) // 2], 5),
        "ms_min": round(per[0], 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else int(traffic["hbm_bytes_per_launch"]),
            "algorithmic_bytes": wl.algorithmic_bytes,
            "kernel": HBM_OPS[op]["key"](wl),
        },
    }


def hbm_op_cpu_baseline(op: str, wl, target_s: float):
    """The oracle on an evenly spaced sample of rows, in algorithmic GB/s."""
    import numpy as np

    import oracle

    run_rows, what = HBM_OPS[op]["oracle_rows"](wl)
    threads = oracle.default_threads()

    def run(n):
        rows = np.linspace(0, wl.rows - 1, n).round().astype(np.int64)
        t0 = time.perf_counter()
        run_rows(rows, threads)
        return time.perf_counter() - t0

    t1 = run(min(wl.rows, 16))
    n = int(min(wl.rows, max(16, round(16 * target_s / max(t1, 1e-6)))))
    t = run(n)
    gbs = wl.algorithmic_bytes * n / wl.rows / t / 1e9
    log(f"[bench] oracle {op}: {n} rows in {t:.2f} s on {threads} threads -> {gbs:.2f} GB/s")
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.rows} rows (evenly spaced), {what}; {t:.2f} s"}


def device_copy_gbs(nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Context for the HBM roof: GB/s (bytes read + written) of torch's own device copy."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] torch device copy of {nbytes >> 20} MiB: {gbs:.0f} GB/s (read + write)")
    return round(gbs, 1)


def _sclk_files():
    return sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))


def _read_sclk_mhz(path):
    """Current shader-clock level (MHz) from a pp_dpm_sclk table (the line marked '*')."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
    except (OSError, ValueError, IndexError):
        return None
    return None


def observed_sclk(w, seconds: float):
    """Median shader clock (MHz) sampled from sysfs while the workload runs untimed.

    The card whose clock is highest during the run is taken as the one in use; None
    when the tables are not readable."""
    import threading

    import torch

    import fa2_fwd_amd as hfa
    from fa2_fwd_amd import workloads as W

    files = _sclk_files()
    if not files:
        return None
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.workload_inputs(w))
    samples = {f: [] for f in files}
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            for f in files:
                mhz = _read_sclk_mhz(f)
                if mhz is not None:
                    samples[f].append(mhz)
            time.sleep(0.005)

    th = threading.Thread(target=sampler, daemon=True)
    ws = attn_workspace(w, dev)
    hfa.attn_fwd(q, k, v, w.scale, workspace=ws)
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            hfa.attn_fwd(q, k, v, w.scale, workspace=ws)
        torch.cuda.synchronize()
    stop.set()
    th.join()
    medians = [sorted(v)[len(v) // 2] for v in samples.values() if v]
    return max(medians) if medians else None


def cpu_baseline(w, target_s: float):
    """The fp64 oracle, as it is, on a bounded sample of query rows of the same workload."""
    import numpy as np

    import oracle
    from fa2_fwd_amd import workloads as W

    qa, ka, va = (W.to_oracle_array(t) for t in W.workload_inputs(w))
    threads = oracle.default_threads()
    heads = w.B * w.H

    def run(rows_per_head):
        rows = np.linspace(0, w.N - 1, rows_per_head).round().astype(np.int64)
        t0 = time.perf_counter()
        oracle.attn_fwd(qa, ka, va, w.scale, rows=rows, threads=threads)
        return time.perf_counter() - t0

    # Two short calibration runs separate the per-head widening cost from the
    # per-row cost; the measured run is then sized to about target_s.
    r0, r1 = min(w.N, 8), min(w.N, 40)
    t0, t1 = run(r0), run(r1)
    per_row = max((t1 - t0) / max(r1 - r0, 1), 1e-6)
    fixed = max(t0 - per_row * r0, 0.0)
    r = int(min(w.N, max(r1, round((target_s - fixed) / per_row))))
    t = run(r)
    flops = 4 * heads * r * w.N * w.d
    value = flops / t / 1e12
    log(f"[bench] oracle: {r} rows/head x {heads} heads in {t:.2f} s on {threads} threads "
        f"-> {value * 1e3:.2f} GFLOP/s")
    return {
        "value": value,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{r} of {w.N} query rows per head (evenly spaced) x {heads} heads, full key length, "
                  f"fp64 definition with the score rows materialised; {t:.2f} s",
    }


def host_info() -> dict:
    """The host the oracle timings ran on: CPU model, logical CPUs, CPUs this process may use."""
    import oracle

    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_usable": usable,
            "oracle_threads": oracle.default_threads()}


def oracle_time(w, threads: int):
    """Seconds the oracle (fp64 definition, score rows materialised) takes for the whole workload."""
    import oracle
    from fa2_fwd_amd import workloads as W

    qa, ka, va = (W.to_oracle_array(t) for t in W.workload_inputs(w))
    t0 = time.perf_counter()
    oracle.attn_fwd(qa, ka, va, w.scale, threads=threads)
    return time.perf_counter() - t0


def oracle_times(configs, main_cfg: int, cpu_main, single_thread=(1, 2, 3)):
    """Oracle seconds per workload: whole workloads on all oracle threads, the small ones
    (`single_thread`) also on one thread; the main workload (too large for the oracle in full)
    by extrapolation from its sampled cpu_baseline."""
    import oracle

    threads = oracle.default_threads()
    out = {}
    for n, wn in sorted(configs.items()):
        if n == main_cfg and wn.flops > 1e12:
            if cpu_main is not None:
                out[n] = {"rows": "sampled (cpu_baseline)", "threads": cpu_main["cores"],
                          "s_extrapolated": round(wn.flops / (cpu_main["value"] * 1e12), 1),
                          "gflops": round(cpu_main["value"] * 1e3, 2)}
            continue
        if wn.flops > 1e12:
            continue
        t = oracle_time(wn, threads)
        entry = {"rows": "all", "threads": threads, "s": round(t, 3), "gflops": round(wn.flops / t / 1e9, 2)}
        if n in single_thread:
            t1 = oracle_time(wn, 1)
            entry.update({"s_1thread": round(t1, 3), "gflops_1thread": round(wn.flops / t1 / 1e9, 2)})
        log(f"[bench] oracle {wn.describe()}: {t:.2f} s on {threads} threads"
            + (f", {entry['s_1thread']:.2f} s on 1" if "s_1thread" in entry else ""))
        out[n] = entry
    return out


def profile_pass_hbm_op(op: str, wl, launches: int) -> None:
    """A few launches of an HBM-bound operation and one device copy of COPY_BYTES, for counter runs."""
    import torch

    launch = HBM_OPS[op]["launcher"](wl)
    stream = torch.cuda.current_stream()
    for _ in range(launches):
        launch(stream)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[profile] {launches} launches of {wl.describe()} and one {COPY_BYTES} B copy done")


def profile_pass(w, launches: int, warmup: int, ramp_s: float) -> None:
    """For counter runs: the timed path's warm-up (W launches, then ramp_s seconds of them),
    `launches` more launches, and one device copy of COPY_BYTES.  The summaries use the last
    `launches` dispatches of the kernel, taken at the clock the timed launches run at."""
    import torch

    import fa2_fwd_amd as hfa
    from fa2_fwd_amd import workloads as W

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.workload_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws = attn_workspace(w, dev)
    warm_up(lambda: hfa.attn_fwd(q, k, v, w.scale, out=o, lse=lse, stream=stream, workspace=ws), warmup, ramp_s)
    for _ in range(launches):
        hfa.attn_fwd(q, k, v, w.scale, out=o, lse=lse, stream=stream, workspace=ws)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[profile] {launches} launches of {w.describe()} and one {COPY_BYTES} B copy done")


def _read_counter(dirpath: str, counter: str):
    """Per-dispatch (kernel name, value) from a rocprofv3 counter_collection.csv."""
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {dirpath}")
    out = []
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter:
                    out.append((int(row.get("Dispatch_Id", 0)), row.get("Kernel_Name", ""),
                                float(row["Counter_Value"])))
    out.sort()
    return [(name, v) for _, name, v in out]


def summarize_pmc(w, fetch_dir: str, write_dir: str, op: str = "attn", last: int = 0) -> None:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the measured kernel (attention, or the
    HBM-bound operation `op`), each scaled by what the same counter reads for the copy of
    known size; over the last `last` dispatches of the kernel (all when 0)."""
    marker = "attn_fwd" if op == "attn" else HBM_OPS[op]["marker"]
    result = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counter(d, counter)
        kern = [v for name, v in rows if marker in name]
        if last > 0:
            kern = kern[-last:]
        # The device-to-device copy is HIP's blit kernel; fall back to the
        # largest other dispatch if the runtime names it differently.
        copies = [v for name, v in rows if "copyBuffer" in name]
        if not copies:
            copies = [v for name, v in rows if marker not in name and v * 1024 > COPY_BYTES * 0.25]
        if not kern or not copies:
            raise RuntimeError(f"{counter}: missing {marker} ({len(kern)}) or copy ({len(copies)}) dispatches")
        copy_kib = max(copies)
        factor = (COPY_BYTES / 1024) / copy_kib
        kib = sum(kern) / len(kern)
        result[counter] = {"kernel_kib_per_dispatch": kib, "copy_kib": copy_kib, "scale": factor,
                           "bytes_per_launch": kib * 1024 * factor}
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    total = result["FETCH_SIZE"]["bytes_per_launch"] + result["WRITE_SIZE"]["bytes_per_launch"]
    key = kernel_key(w) + f"_N{w.N}" if op == "attn" else HBM_OPS[op]["key"](w)
    alg = algorithmic_bytes(w) if op == "attn" else w.algorithmic_bytes
    table[key] = {
        "workload": w.describe(),
        "src_digest": kernel_source_digest(op),
        "fetch": result["FETCH_SIZE"],
        "write": result["WRITE_SIZE"],
        "hbm_bytes_per_launch": total,
        "algorithmic_bytes": alg,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=2, sort_keys=True)
        f.write("\n")
    log(f"[pmc] {w.describe()}: HBM {total / 1e6:.1f} MB/launch vs algorithmic {alg / 1e6:.1f} MB")


def _csv_rows(dirpath: str, suffix: str):
    files = glob.glob(os.path.join(dirpath, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    rows = []
    for path in files:
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _last_json_line(path: str):
    with open(path) as f:
        lines = [ln for ln in f if ln.strip().startswith("{")]
    return json.loads(lines[-1])


def _config_ms(line: dict, n: int):
    """ms_per_step of workload n in a bench JSON line (headline, secondary or all_configs)."""
    for e in line.get("all_configs") or []:
        if e["config"] == n:
            return e["ms_per_step"]
    if line.get("config", {}).get("workload") == W_describe(n):
        return line["ms_per_step"]
    sec = line.get("secondary")
    if sec and sec["config"]["workload"] == W_describe(n):
        return sec["ms_per_step"]
    return None


def W_describe(n: int) -> str:
    from fa2_fwd_amd import workloads as W

    return W.CONFIGS[n].describe()


def kernel_profile_name(w) -> str:
    return f"attn_fwd_{w.dtype}_d{w.d}_N{w.N}"


def summarize_trace(n: int, trace_dir: str, trace_json: str, bench_json: str | None, command: str) -> None:
    """profiles/<kernel>.md: kernel durations of a traced run of the timed path, beside the
    event timing of that run and the unprofiled bench run of the same job."""
    from fa2_fwd_amd import workloads as W

    w = W.CONFIGS[n]
    traced = _last_json_line(trace_json)
    steps = int(traced["steps"])
    rows = [r for r in _csv_rows(trace_dir, "kernel_trace.csv") if "attn_fwd" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    timed = durs[-steps:]
    avg_timed = sum(timed) / len(timed)
    st = [r for r in _csv_rows(trace_dir, "kernel_stats.csv") if "attn_fwd" in r["Name"]][0]
    traced_ms = float(traced["ms_per_step"])
    bench_ms = None
    if bench_json:
        bench_ms = _config_ms(_last_json_line(bench_json), n)
    tflops_trace = w.flops / (avg_timed * 1e-9) / 1e12
    roof = traced["roofline"]
    frac_trace = tflops_trace / roof["peak"]
    traffic = load_traffic(w)
    lines = [f"# {kernel_profile_name(w)} -- {w.describe()}", "",
             "## Kernel time (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{command}`", "",
             f"The traced process runs the timed path of `bench.py`: {traced['warmup']} warm-up launches, "
             f"{traced['warm_s']} s more of them (clock ramp), then {steps} timed launches between HIP events. "
             f"The last {steps} dispatches of the kernel in the trace are those timed launches.", "",
             "| kernel | calls (all) | avg ns (all) | min ns | max ns |", "|---|---|---|---|---|",
             f"| `{st['Name'][:100]}` | {st['Calls']} | {float(st['AverageNs']):.0f} | {st['MinNs']} | {st['MaxNs']} |",
             "", "| figure | ms |", "|---|---|",
             f"| trace: average duration of the {steps} timed dispatches | {avg_timed / 1e6:.5f} |",
             f"| the traced run's own event timing (`ms_per_step` of its JSON line) | {traced_ms:.5f} |"]
    if bench_ms is not None:
        lines.append(f"| unprofiled `python bench.py` in the same job (`ms_per_step` of this workload) | {bench_ms:.5f} |")
    # other kernels of each step (the fp32 packing kernel, the bf16 key-split merge)
    others = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if "attn_fwd" not in name and ("f32_pack_kernel" in name or "attn_merge" in name):
            others.setdefault(name, []).append(r)
    step_total = avg_timed
    for name, rs in sorted(others.items()):
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        od = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs][-steps:]
        avg_o = sum(od) / len(od)
        step_total += avg_o
        lines.append(f"| trace: average of the last {len(od)} dispatches of `{name.split('(')[0][:80]}` (same step) "
                     f"| {avg_o / 1e6:.5f} |")
    if others:
        lines.append(f"| trace: the step's kernels together | {step_total / 1e6:.5f} |")
    lines += ["",
              f"From the trace: {tflops_trace:.1f} TFLOP/s = {frac_trace:.4f} of the {roof['peak']} TFLOP/s "
              f"roofline (the line: {roof['achieved']} TFLOP/s, frac {roof['frac']}).",
              f"Trace average / event ms_per_step of the traced run: {avg_timed / 1e6 / traced_ms:.4f}"
              + (f"; / unprofiled ms_per_step: {avg_timed / 1e6 / bench_ms:.4f}." if bench_ms else "."), ""]
    if others:
        lines += [f"The step also runs the kernels listed after the attention kernel; all of them together: "
                  f"{step_total / 1e6 / traced_ms:.4f} of the traced run's ms_per_step"
                  + (f", {step_total / 1e6 / bench_ms:.4f} of the unprofiled one." if bench_ms else "."), ""]
    if traffic is not None:
        t = traffic
        lines += ["## HBM bytes (rocprofv3 --pmc, one counter per run)", "",
                  f"Commands: `rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch{n} -o run --output-format csv -- "
                  f"python bench.py --profile-pass --config {n}` and the same with `WRITE_SIZE` into "
                  f"`gpurun_out/pmc_write{n}`; then `python bench.py --summarize-pmc gpurun_out/pmc_fetch{n} "
                  f"gpurun_out/pmc_write{n} --config {n}`.",
                  f"Each counter is scaled by what it reads for a plain 512 MiB device copy in the same run "
                  f"(FETCH_SIZE x{t['fetch']['scale']:.4f}, WRITE_SIZE x{t['write']['scale']:.4f}).", "",
                  "| counter | KiB/dispatch (raw) | copy KiB (raw, 524288 expected) | scaled bytes/launch |",
                  "|---|---|---|---|",
                  f"| FETCH_SIZE | {t['fetch']['kernel_kib_per_dispatch']:.1f} | {t['fetch']['copy_kib']:.1f} | "
                  f"{t['fetch']['bytes_per_launch']:.0f} |",
                  f"| WRITE_SIZE | {t['write']['kernel_kib_per_dispatch']:.1f} | {t['write']['copy_kib']:.1f} | "
                  f"{t['write']['bytes_per_launch']:.0f} |", "",
                  f"HBM traffic per launch: {t['hbm_bytes_per_launch'] / 1e6:.1f} MB; algorithmic (Q, K, V read "
                  f"once, O and LSE written once): {t['algorithmic_bytes'] / 1e6:.1f} MB.",
                  f"Over the traced average kernel time: {t['hbm_bytes_per_launch'] / avg_timed:.1f} GB/s of counted "
                  f"traffic ({t['hbm_bytes_per_launch'] / avg_timed / HBM_PEAK_GBS:.3f} of the {HBM_PEAK_GBS:.0f} GB/s "
                  f"HBM peak), {t['algorithmic_bytes'] / avg_timed:.1f} GB/s of algorithmic bytes.", ""]
    lines.append(f"Kernel source digest when taken: `{kernel_source_digest()}`.")
    path = os.path.join(ROOT, "profiles", kernel_profile_name(w) + ".md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[profile] {path}: trace {avg_timed / 1e6:.5f} ms vs event {traced_ms:.5f} ms"
        + (f" vs bench {bench_ms:.5f} ms" if bench_ms else ""))


SQ_GROUPS = (
    "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
    "SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES",
    "GRBM_GUI_ACTIVE SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS "
    "SQ_INSTS_VALU_TRANS_F32 SQ_ACTIVE_INST_ANY SQ_INSTS_SALU",
)


def summarize_sq(n: int, sq1: str, sq2: str, trace_dir: str, launches: int) -> None:
    """profiles/<kernel>_sq.md from two shader-counter runs and a kernel trace of --profile-pass,
    each over the last `launches` dispatches (after the timed path's warm-up)."""
    from fa2_fwd_amd import workloads as W

    w = W.CONFIGS[n]
    vals: dict[str, list[float]] = {}
    for d in (sq1, sq2):
        per: dict[str, dict[int, float]] = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if "attn_fwd" in r["Kernel_Name"]:
                per.setdefault(r["Counter_Name"], {})[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
        for name, by_id in per.items():
            last = [by_id[i] for i in sorted(by_id)[-launches:]]
            vals.setdefault(name, []).extend(last)
    c = {k: sum(v) / len(v) for k, v in vals.items()}
    rows = sorted((r for r in _csv_rows(trace_dir, "kernel_trace.csv") if "attn_fwd" in r["Kernel_Name"]),
                  key=lambda r: int(r["Dispatch_Id"]))
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows][-launches:]
    avg_us = sum(durs) / len(durs) / 1e3
    act = c["GRBM_GUI_ACTIVE"] / 8
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * act)
    pp = f"python bench.py --profile-pass --config {n} --launches {launches}"
    lines = [f"# {kernel_profile_name(w)}_sq -- shader counters, {w.describe()}", "",
             f"Each run: `{pp}` (the timed path's warm-up, then {launches} launches and one 512 MiB copy); "
             f"figures are averages over the last {launches} dispatches of the kernel.", "",
             f"- `rocprofv3 --pmc {SQ_GROUPS[0]} -d gpurun_out/sq1_c{n} -o run --output-format csv -- {pp}`",
             f"- `rocprofv3 --pmc {SQ_GROUPS[1]} -d gpurun_out/sq2_c{n} -o run --output-format csv -- {pp}`",
             f"- `rocprofv3 --kernel-trace --stats -d gpurun_out/sqtr_c{n} -o run --output-format csv -- {pp}`", "",
             "| counter (per launch, whole chip) | value |", "|---|---|"]
    for k in sorted(c):
        lines.append(f"| {k} | {c[k]:.4g} |")
    lds = max(c.get("SQ_INSTS_LDS", 0.0), 1.0)
    lines += ["", f"Kernel time under the trace (last {launches} dispatches): {avg_us:.1f} us.", "", "Derived:", "",
              f"- GPU-active cycles per XCD: {act:.4g}, i.e. {act / (avg_us * 1e3):.2f} GHz over the traced time "
              f"(counter and trace runs are separate processes).",
              f"- Matrix-core busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x active cycles) = {100 * busy:.1f} %.",
              f"- MFMA instructions: {c['SQ_INSTS_MFMA']:.4g}; LDS instructions: {c['SQ_INSTS_LDS']:.4g}; LDS "
              f"bank-conflict cycles: {c['SQ_LDS_BANK_CONFLICT']:.4g} ({c['SQ_LDS_BANK_CONFLICT'] / lds:.3f} per LDS "
              f"instruction).",
              f"- VALU instructions: {c['SQ_INSTS_VALU']:.4g}, of which transcendental (exp) "
              f"{c['SQ_INSTS_VALU_TRANS_F32']:.4g}; SALU {c['SQ_INSTS_SALU']:.4g}.",
              f"- MFMA cycles with VALU issued alongside: "
              f"{100 * c['SQ_VALU_MFMA_COEXEC_CYCLES'] / max(c['SQ_VALU_MFMA_BUSY_CYCLES'], 1):.1f} % of MFMA busy "
              f"cycles.", "", f"Kernel source digest when taken: `{kernel_source_digest()}`.", ""]
    path = os.path.join(ROOT, "profiles", kernel_profile_name(w) + "_sq.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    log(f"[profile] {path}: {avg_us:.1f} us, MFMA busy {100 * busy:.1f} %, LDS conflicts per LDS instruction "
        f"{c['SQ_LDS_BANK_CONFLICT'] / lds:.3f}")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5, help="workload number 1-5 (default 5)")
    ap.add_argument("--secondary", type=int, default=3, help="second workload timed beside it (0: none)")
    ap.add_argument("--no-all-configs", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--no-sclk", action="store_true", help="skip sampling the shader clock")
    ap.add_argument("--cpu-seconds", type=float, default=14.0,
                    help="target oracle time for cpu_baseline (the sizing from short runs lands near 70%% of it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", action="store_true")
    ap.add_argument("--launches", type=int, default=5, help="--profile-pass: launches after the warm-up")
    ap.add_argument("--ramp-s", type=float, default=CLOCK_RAMP_S,
                    help="seconds of untimed launches after the W warm-up launches (clock ramp)")
    ap.add_argument("--no-oracle-times", action="store_true",
                    help="skip the oracle timings of the small workloads (all_configs[].oracle)")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/<kernel>.md from a rocprofv3 --kernel-trace --stats run of this "
                         "command's timed path (see --trace-json, --bench-json)")
    ap.add_argument("--trace-json", help="--summarize-trace: the JSON line printed by the traced run")
    ap.add_argument("--bench-json", help="--summarize-trace: the JSON line of the unprofiled bench run "
                                         "of the same job")
    ap.add_argument("--summarize-sq", nargs=3, metavar=("SQ1_DIR", "SQ2_DIR", "TRACE_DIR"),
                    help="write profiles/<kernel>_sq.md from two shader-counter runs of --profile-pass "
                         "and a kernel trace of the same pass")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--op", choices=("attn", "softmax", "rmsnorm"), default="attn",
                    help="kernel for --profile-pass / --summarize-pmc / --op-only (--config numbers that "
                         "op's workloads)")
    ap.add_argument("--op-only", action="store_true", help="time only workload --config of --op")
    ap.add_argument("--softmax-only", action="store_true", help="same as --op softmax --op-only")
    ap.add_argument("--no-softmax", action="store_true", help="skip the row softmax workloads")
    ap.add_argument("--no-rmsnorm", action="store_true", help="skip the RMS normalisation workloads")
    args = ap.parse_args()

    from fa2_fwd_amd import workloads as W

    if args.softmax_only:
        args.op, args.op_only = "softmax", True
    if args.op != "attn" and (args.summarize_pmc or args.profile_pass):
        wl = hbm_configs(args.op)[args.config]
        if args.summarize_pmc:
            summarize_pmc(wl, *args.summarize_pmc, op=args.op)
        else:
            profile_pass_hbm_op(args.op, wl, args.launches)
        return 0
    w = W.CONFIGS[args.config]
    if args.summarize_pmc:
        summarize_pmc(w, *args.summarize_pmc, last=args.launches)
        return 0
    if args.summarize_trace:
        traced_cmd = (f"rocprofv3 --kernel-trace --stats -d {args.summarize_trace} -o run --output-format csv -- "
                      f"python bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} "
                      f"--secondary 0 --no-all-configs --no-sclk --no-softmax --no-rmsnorm --no-cpu-baseline")
        summarize_trace(args.config, args.summarize_trace, args.trace_json, args.bench_json, traced_cmd)
        return 0
    if args.summarize_sq:
        summarize_sq(args.config, *args.summarize_sq, args.launches)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this attention forward is a single-GPU kernel; "
              "see the design notes for how it would shard across GPUs.", file=sys.stderr)
        return 2
    if args.profile_pass:
        profile_pass(w, args.launches, args.warmup, args.ramp_s)
        return 0

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.op_only:
        if args.op == "attn":
            print("--op-only needs --op softmax or --op rmsnorm", file=sys.stderr)
            return 2
        print(json.dumps(time_hbm_op(args.op, hbm_configs(args.op)[args.config], args.steps, args.warmup)),
              flush=True)
        return 0
    main_res = time_gpu(w, args.steps, args.warmup, args.ramp_s)
    secondary = None
    if args.secondary and args.secondary != args.config:
        w2 = W.CONFIGS[args.secondary]
        r2 = time_gpu(w2, args.steps, args.warmup, args.ramp_s)
        secondary = {
            "metric": "attention fwd TFLOP/s",
            "value": round(r2["tflops"], 3),
            "unit": "TFLOP/s",
            "ms_per_step": round(r2["ms"], 5),
            "dtype": w2.dtype,
            "arith": ARITH[w2.dtype],
            "config": {"workload": w2.describe(), "B": w2.B, "H": w2.H, "N": w2.N, "d": w2.d},
            "roofline": r2["roofline"],
            "cpu_baseline": None,
        }
    all_configs = None
    if not args.no_all_configs:
        all_configs = []
        for n in sorted(W.CONFIGS):
            if n == args.config:
                r = main_res
            elif secondary is not None and n == args.secondary:
                r = r2
            else:
                r = time_gpu(W.CONFIGS[n], max(10, args.steps // 2), args.warmup, args.ramp_s)
            wn = W.CONFIGS[n]
            graph_ms = graph_time(wn, 100, 3) if wn.flops < 1e10 else None
            if graph_ms is not None:
                log(f"[bench] {wn.describe()}: {graph_ms * 1e3:.2f} us/launch replayed from a graph of 100")
            entry = {
                "config": n, "workload": wn.describe(), "dtype": wn.dtype,
                "ms_per_step": round(r["ms"], 5), "ms_median": round(r["ms_median"], 5),
                "ms_min": round(r["ms_min"], 5), "tflops": round(r["tflops"], 3),
                "peak": r["roofline"]["peak"], "frac_of_peak": r["roofline"]["frac"],
                "ms_per_launch_graph": None if graph_ms is None else round(graph_ms, 5),
            }
            if wn.dtype == "f32":
                entry["fp32_frac"] = r["roofline"]["fp32_frac"]
            all_configs.append(entry)
    sclk = None if args.no_sclk else observed_sclk(w, 0.5)
    if sclk is not None:
        log(f"[bench] shader clock during {w.describe()}: {sclk:.0f} MHz (median of sysfs samples)")
    copy_gbs = None if (args.no_softmax and args.no_rmsnorm) else device_copy_gbs()
    hbm = {}
    for op, skip, baseline_cfg in (("softmax", args.no_softmax, 1), ("rmsnorm", args.no_rmsnorm, 3)):
        if skip:
            continue
        entries = []
        for n, wl in sorted(hbm_configs(op).items()):
            entry = time_hbm_op(op, wl, args.steps, args.warmup)
            entry["config"] = n
            if n == baseline_cfg and not args.no_cpu_baseline:
                entry["cpu_baseline"] = hbm_op_cpu_baseline(op, wl, 3.0)
            entries.append(entry)
        hbm[HBM_OPS[op]["json_key"]] = entries
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    host = None
    if not args.no_cpu_baseline:
        host = host_info()
        log(f"[bench] host: {host}")
    if not args.no_cpu_baseline and not args.no_oracle_times:
        otimes = oracle_times(W.CONFIGS, args.config, cpu)
        for entry in all_configs or []:
            entry["oracle"] = otimes.get(entry["config"])
        if secondary is not None and args.secondary in otimes and "s" in otimes[args.secondary]:
            o2 = otimes[args.secondary]
            secondary["cpu_baseline"] = {
                "value": round(W.CONFIGS[args.secondary].flops / o2["s"] / 1e12, 6), "unit": "TFLOP/s",
                "cores": o2["threads"], "kind": "oracle",
                "sample": f"the whole workload (every query row of every head), fp64 definition with the score "
                          f"rows materialised; {o2['s']:.2f} s",
            }
    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d per launch) and fraction of MFMA peak",
        "value": round(main_res["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_s": args.ramp_s,
        "ms_per_step": round(main_res["ms"], 5),
        "ms_median": round(main_res["ms_median"], 5),
        "ms_min": round(main_res["ms_min"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "arith": ARITH[w.dtype],
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": w.describe(), "B": w.B, "H": w.H, "N": w.N, "d": w.d, "seed": w.seed},
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
        "all_configs": all_configs,
        "softmax_rows": hbm.get("softmax_rows"),
        "rmsnorm": hbm.get("rmsnorm"),
        "device_copy_gbs": copy_gbs,
        "observed_sclk_mhz": sclk,
        "device": getattr(props, "gcnArchName", props.name),
        "host": host,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
