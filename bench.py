#!/usr/bin/env python3
"""Benchmark of the fused attention forward (libmifa) on one MI355X.

One step = one mifa_fwd launch over one batch of the workload (default: B=1, H=32, N=16384,
d=128, causal, bf16 Q/K/V ~ N(0,1), the long-context configuration the throughput target is
quoted on).  Inputs are generated with a seeded CPU generator and are resident in HBM before
the timed region.  Prints ONE JSON line on stdout.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4] [--no-cpu-baseline]

FLOPs per step follow the usual attention convention: 4*B*H*N^2*d, halved for causal.

Warm-up: --warmup W runs exactly W untimed launches; without it, at least 30 launches and at
least 0.5 s of them, and the JSON line reports the count that ran.

`--workload D1` / `D2` time the split-KV path (mifa_attention_splitkv) on few queries against a
long key/value cache; the metric is HBM throughput of the compulsory bytes (Q, K, V read once,
O and LSE written once).

`--workload SM1` .. `SM5` time the stand-alone row softmax (mifa_softmax_rows) instead: one
step is one launch over a [rows, cols] matrix, and the metric is HBM throughput of the
compulsory bytes (the input read once, the output and the row LSE written once).

`--workload GEMM-ref` times the vendor library's bf16 GEMM (torch.matmul, M = N = K = 8192) with
its sustained clock, for context: what a plain contraction reaches on the same GPU.  Likewise
`--workload HBM-ref` times the runtime's 1 GiB device copy (and a 2 GiB torch.sum), the vendor's
streaming rates the HBM-bound legs read against.  Neither is this library's code; neither has a CPU
baseline.

Besides the driver's fields, `roofline` and `cpu_baseline`, the line carries `provenance` (source
hashes, git commit where available, GPU, ROCm/HIP/torch versions, seed); on the attention legs
`clock`, the sustained engine clock measured on the GPU by short mifa_clock_probe runs during a
further second of untimed launches after the timed ones, and the percentage of the peak at that
clock; and on the forward
legs `parity`, the errors of the last timed launch's O and LSE on the rows the CPU-baseline leg
computed with the float64 oracle.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # 312.5
LLC_BYTES = 256 << 20      # MI355X last-level (Infinity) cache
KERNEL_SOURCE = os.path.join(ROOT, "io_aware_softmax_mifa_amd", "csrc", "mifa_fwd.hip")
BWD_SOURCE = os.path.join(ROOT, "io_aware_softmax_mifa_amd", "csrc", "mifa_bwd.hip")
SOFTMAX_SOURCE = os.path.join(ROOT, "io_aware_softmax_mifa_amd", "csrc", "mifa_softmax.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


MIN_WARMUP_STEPS = 30
WARMUP_SECONDS = 0.5


def warm_up(step, requested) -> int:
    """Untimed warm-up launches; returns how many ran.  With --warmup W exactly W; by default at
    least MIN_WARMUP_STEPS launches and at least WARMUP_SECONDS of wall time, so that the GPU
    clock has left its idle state before the timed region (short workloads otherwise finish
    their warm-up within milliseconds)."""
    import torch

    if requested is not None:
        for _ in range(requested):
            step()
        torch.cuda.synchronize()
        return requested
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if n >= MIN_WARMUP_STEPS and time.perf_counter() - t0 >= WARMUP_SECONDS:
            return n


def forward_roofline(f: float, cb: int, kernel_ms: float) -> dict:
    """Roofline entry of a forward leg: the bound the arithmetic intensity implies.  Below the
    ridge (peak FLOP/s over peak HBM bytes/s, 312.5 FLOP/B) the compulsory bytes per second
    against 8 TB/s; at or above it the FLOPs per second against 2.5 PFLOP/s."""
    if f / cb >= RIDGE_FLOP_PER_BYTE:
        achieved = f / (kernel_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    gbs = cb / (kernel_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS}


def flops(w) -> float:
    f = 4.0 * w.B * w.H * w.N * w.N * w.d
    return f / 2 if w.causal else f


def compulsory_bytes(w) -> int:
    """bf16 Q, K, V read once; fp32 O and LSE written once."""
    n = w.B * w.H * w.N
    return 3 * 2 * n * w.d + 4 * n * w.d + 4 * n


def kernel_sha(source: str = KERNEL_SOURCE) -> str:
    with open(source, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, source: str = KERNEL_SOURCE):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    counters were taken on another kernel source or another workload.  An entry may carry its
    own source hash (other kernels than the attention forward)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload)
    if not entry:
        return None
    if entry.get("kernel_source_sha256", t.get("kernel_source_sha256")) != kernel_sha(source):
        return None
    return entry.get("traffic_bytes")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def host_info() -> dict:
    """What the oracle ran on: logical CPUs, the ones this process may use, the CPU model."""
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
    except (AttributeError, OSError):
        usable = None
    return {"host_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


PEAK_CLOCK_MHZ = 2400.0    # MI355X peak engine clock, the clock the 2.5 PFLOP/s figure assumes
CLOCK_WINDOW_S = 1.0       # untimed launches after the timed steps, during which the clock is measured
CLOCK_SETTLE_S = 0.25      # into that window, when the first clock probe starts
CLOCK_SPAN_US = 20         # each probe's span: short, since a probe wave holds a slot on its CU
CLOCK_PROBE_GAP_S = 0.015  # at least this long between two probes
CLOCK_MAX_PROBES = 40


def sample_clock(step, value_tflops):
    """The sustained engine clock under this workload, measured on the GPU.  After the timed
    region (untimed, not part of `value`) the same step keeps running for CLOCK_WINDOW_S
    seconds; from CLOCK_SETTLE_S on, every CLOCK_PROBE_GAP_S or more, mifa_clock_probe runs 8
    single-wave probes on a second stream that read the shader-clock and real-time counters
    CLOCK_SPAN_US apart.  Short probes: a kernel that fills every CU's registers cannot place a
    workgroup beside a probe wave, so a long probe would take CUs away from the workload it
    measures (a 20 us probe every 15 ms or more holds 8 CUs for well under 1% of the window).
    Returns the median over all probes and, for a compute-bound leg, the bf16 peak scaled to it
    and `value_tflops` as a percentage of it."""
    import torch

    from io_aware_softmax_mifa_amd import binding

    out = {"source": (f"mifa_clock_probe: groups of 8 single-wave probes on a second stream, each reading "
                      f"s_memtime and s_memrealtime {CLOCK_SPAN_US} us apart, one group every "
                      f">= {CLOCK_PROBE_GAP_S * 1e3:g} ms from {CLOCK_SETTLE_S:g} s into {CLOCK_WINDOW_S:g} s of "
                      f"further launches of the same step after the timed steps"),
           "probes": 0, "median_mhz": None, "min_mhz": None, "max_mhz": None, "error": None}
    buf = torch.zeros(CLOCK_MAX_PROBES * 32, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()  # default priority; non-blocking with respect to the null stream
    khz, n, last, prev = 0, 0, None, None
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_WINDOW_S:
        for _ in range(5):
            step()
        ev = torch.cuda.Event()
        ev.record()
        if prev is not None:
            prev.synchronize()  # keep about one group of steps queued behind the running one
        prev = ev
        now = time.perf_counter() - t0
        if (now >= CLOCK_SETTLE_S and n < CLOCK_MAX_PROBES and (last is None or now - last >= CLOCK_PROBE_GAP_S)
                and now + 2 * CLOCK_PROBE_GAP_S < CLOCK_WINDOW_S):
            st, khz = binding.mifa_clock_probe_raw(buf[32 * n:], CLOCK_SPAN_US, side.cuda_stream)
            if st != 0:
                out["error"] = f"mifa_clock_probe: {binding.mifa_status_string(st)}"
                break
            n, last = n + 1, now
    torch.cuda.synchronize()
    out["probes"] = n
    if out["error"] is None and n == 0:
        out["error"] = "no probe was launched"
    if out["error"] is None:
        v = buf[:32 * n].cpu().tolist()
        mhz = []
        for w in range(8 * n):
            dt, dr = v[4 * w + 2] - v[4 * w], v[4 * w + 3] - v[4 * w + 1]
            mhz.append(dt / dr * khz / 1e3 if dr > 0 else float("nan"))
        if not all(100.0 < x < 3000.0 for x in mhz):
            out["error"] = "probe clock outside 100..3000 MHz"
        else:
            srt = sorted(mhz)
            out.update(median_mhz=srt[len(srt) // 2], min_mhz=srt[0], max_mhz=srt[-1])
            if value_tflops is not None:
                peak = PEAK_BF16_TFLOPS * out["median_mhz"] / PEAK_CLOCK_MHZ
                out["clock_adjusted_peak_tflops"] = peak
                out["pct_of_clock_adjusted_peak"] = 100.0 * value_tflops / peak
    return out


SOURCES = [os.path.join(ROOT, "io_aware_softmax_mifa_amd", "csrc", f)
           for f in ("mifa_fwd.hip", "mifa_bwd.hip", "mifa_softmax.hip", "mifa_clock.hip", "mifa_common.h")]


def provenance(seed) -> dict:
    """What produced this line: source hashes, git commit (where the checkout has .git), GPU and
    software versions, and the workload's seed.  The GPU's name is amdsmi's market name, else
    the HIP device name (which can be a generic one)."""
    import subprocess

    import torch

    h = hashlib.sha256()
    for path in SOURCES + [os.path.abspath(__file__)]:
        with open(path, "rb") as f:
            h.update(f.read())
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        sha = None
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    name, name_err = None, None
    try:
        import amdsmi

        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        try:
            handles = amdsmi.amdsmi_get_processor_handles()
            if handles:
                name = amdsmi.amdsmi_get_gpu_asic_info(handles[0]).get("market_name") or None
                if not name:
                    name = amdsmi.amdsmi_get_gpu_board_info(handles[0]).get("product_name") or None
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # noqa: BLE001 -- the name is informational
        name, name_err = None, repr(e)[:200]
    name = name or torch.cuda.get_device_name(0) or None
    from io_aware_softmax_mifa_amd import binding

    return {"git_sha": sha, "sources_sha256": h.hexdigest()[:16], "gpu_name": name,
            "gpu_arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "rocm_version": rocm, "hip_runtime": torch.version.hip, "torch_version": torch.__version__,
            "library": binding.mifa_version(), "seed": seed,
            **({"gpu_name_note": f"amdsmi: {name_err}; HIP device name used"} if name_err else {})}


def event_stats(starts, ends) -> dict:
    """Median and minimum per-call milliseconds from paired HIP events."""
    ms = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    return {"call_ms_median": ms[len(ms) // 2], "call_ms_min": ms[0]}


def cpu_baseline(w, q, k, v, scale, rows_count: int, o_gpu=None, lse_gpu=None):
    """The float64 oracle as it stands, timed on this host on a bounded sample of rows.  With the
    timed launch's outputs (o_gpu, lse_gpu on the host) the same oracle rows also give that
    launch's parity: O max/mean-abs and LSE max-abs error on the sampled rows."""
    import numpy as np

    from io_aware_softmax_mifa_amd import workloads as W
    from oracle import attention_fp64_rows

    rows = W.sample_rows(w.B, w.H, w.N, rows_count, w.seed + 7)
    t0 = time.perf_counter()
    ro, rl = attention_fp64_rows(q, k, v, rows, causal=w.causal, scale=scale)
    dt = time.perf_counter() - t0
    parity = None
    if o_gpu is not None:
        r = rows.numpy()
        err = np.abs(o_gpu[r[:, 0], r[:, 1], r[:, 2]].double().numpy() - ro)
        lerr = np.abs(lse_gpu[r[:, 0], r[:, 1], r[:, 2]].double().numpy() - rl)
        parity = {"rows": int(r.shape[0]), "o_max_abs": float(err.max()), "o_mean_abs": float(err.mean()),
                  "lse_max_abs": float(lerr.max()), "bar": {"o_max_abs": 2e-2, "o_mean_abs": 2e-3, "lse_max_abs": 1e-3}}
        parity["pass"] = bool(parity["o_max_abs"] <= 2e-2 and parity["o_mean_abs"] <= 2e-3
                              and parity["lse_max_abs"] <= 1e-3)
    # Credit each sampled row with the per-row share of the step's FLOP convention.
    per_row = flops(w) / (w.B * w.H * w.N)
    value = rows.shape[0] * per_row / dt / 1e12
    out = {
        "value": value,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{rows.shape[0]} seeded query rows of the same workload (float64 NumPy oracle, full "
                   f"score row per query), {dt:.2f} s; credited {per_row:.3e} FLOP per row"),
        "seconds": dt,
        # every row costs the oracle the same (it scores the full row, then masks), so the whole
        # workload would take about this long: an extrapolation, not a run
        "extrapolated_full_oracle_seconds": dt * (w.B * w.H * w.N) / rows.shape[0],
    }
    out.update(host_info())
    return out, parity


def copy_calibration(dev):
    """A plain device-to-device copy of 1 GiB, three times: its FETCH_SIZE / WRITE_SIZE counters
    give the scale from counter units to bytes."""
    import torch

    n = 1 << 29
    a = torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {2 * n} bytes")
    del a, b


def softmax_bytes(w) -> int:
    """Compulsory bytes of one row-softmax launch: x read once, y and lse written once."""
    return 2 * w.rows * w.cols * w.element_bytes + 4 * w.rows


def softmax_cpu_baseline(w, x, rows_count: int):
    """The float64 softmax oracle as it stands, on a bounded seeded sample of rows."""
    from io_aware_softmax_mifa_amd import workloads as W
    from oracle import softmax_rows_fp64

    # rows_count <= 0: every row of the workload (a few seconds of CPU work at these sizes),
    # fed to the oracle in chunks of 16,384 rows to bound host memory
    rows = W.sample_softmax_rows(w.rows, rows_count if rows_count > 0 else w.rows, w.seed + 7)
    t0 = time.perf_counter()
    for i in range(0, rows.shape[0], 16384):
        softmax_rows_fp64(x[rows[i:i + 16384]], w.scale)
    dt = time.perf_counter() - t0
    per_row = softmax_bytes(w) / w.rows
    return {
        "value": rows.shape[0] * per_row / dt / 1e9,
        "unit": "GB/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{rows.shape[0]} of the workload's {w.rows} rows (float64 NumPy oracle), {dt:.2f} s; "
                   f"credited {per_row:.0f} compulsory bytes per row"),
        "seconds": dt,
        **host_info(),
    }


def decode_bytes(w) -> int:
    """Compulsory bytes of one split-KV launch: bf16 Q, K, V read once, fp32 O and LSE written."""
    return 2 * w.B * w.H * (w.Nq + 2 * w.Nk) * w.d + 4 * w.B * w.H * w.Nq * (w.d + 1)


def decode_flops(w) -> float:
    """4 d FLOPs per (query, visible key) pair."""
    if not w.causal:
        pairs = w.Nq * w.Nk
    else:
        pairs = sum(w.Nk - w.Nq + 1 + i for i in range(w.Nq))
    return 4.0 * w.B * w.H * pairs * w.d


def bench_decode(args):
    import torch

    from io_aware_softmax_mifa_amd import binding
    from io_aware_softmax_mifa_amd import workloads as W

    w = W.decode_by_name(args.workload)
    log(f"workload {w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} causal={w.causal}")
    q, k, v = W.make_rect_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.seed, w.dist)
    scale = W.fp32_scale(w.d)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dq, dk, dv = (t.to(dev) for t in (q, k, v))
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    need = binding.mifa_splitkv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        st = binding.mifa_attention_splitkv_raw(dq, dk, dv, o, lse, w.B, w.H, w.Nq, w.Nk, w.d, w.causal, scale, ws,
                                                ws.numel(), stream.cuda_stream)
        if st != 0:
            raise binding.MifaError(st, binding.mifa_status_string(st))

    args.warmup = warm_up(step, args.warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    call_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    if args.copy_calibration:
        copy_calibration(dev)
    nbytes = decode_bytes(w)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {call_ms:.4f} ms/call (HIP events; both kernels)")
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    out = {
        "metric": "attention decode (split-KV) HBM throughput (compulsory bytes) and % of MI355X HBM bandwidth",
        "value": nbytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. bf16 Q/K/V)",
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} causal={int(w.causal)} bf16 "
                        f"Q,K,V ~ N(0,1); fp32 O + LSE; split-KV + merge",
            "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": bool(w.causal),
            "compulsory_hbm_bytes": nbytes,
            "flop_per_step": decode_flops(w),
            "call_ms": call_ms,
            "workspace_bytes": need,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic(w.name, KERNEL_SOURCE),
        },
    }
    out["provenance"] = provenance(w.seed)
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        from oracle import attention_fp64_rows

        rows = torch.tensor([[b, h, i] for b in range(w.B) for h in range(w.H) for i in range(w.Nq)])
        t0 = time.perf_counter()
        attention_fp64_rows(q, k, v, rows, causal=w.causal, scale=scale)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {
            "value": nbytes / dt / 1e9,
            "unit": "GB/s",
            "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"every one of the {rows.shape[0]} query rows (float64 NumPy oracle), {dt:.2f} s",
            "seconds": dt,
            **host_info(),
        }
    out["config"].update(event_stats(starts, ends))
    print(json.dumps(out), flush=True)


def bench_softmax(args):
    import torch

    from io_aware_softmax_mifa_amd import binding
    from io_aware_softmax_mifa_amd import workloads as W

    w = W.softmax_by_name(args.workload)
    log(f"workload {w.name}: rows={w.rows} cols={w.cols} dtype={w.dtype} std={w.std}")
    x = W.make_softmax_input(w.rows, w.cols, w.dtype, w.std, w.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dx = x.to(dev)
    y = torch.empty_like(dx)
    lse = torch.empty(w.rows, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dtype = binding.MIFA_DTYPE_BF16 if w.dtype == "bf16" else binding.MIFA_DTYPE_F32

    def step():
        binding.mifa_softmax_rows(dx, y, lse, w.rows, w.cols, dtype, w.scale, stream.cuda_stream)

    args.warmup = warm_up(step, args.warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    nbytes = softmax_bytes(w)
    if args.copy_calibration:
        copy_calibration(dev)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {kernel_ms:.4f} ms/launch (HIP events)")
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    out = {
        "metric": "row softmax HBM throughput (compulsory bytes) and % of MI355X HBM bandwidth",
        "value": nbytes / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic (seeded i.i.d. normal rows)",
        "config": {
            "workload": f"{w.name}: rows={w.rows} cols={w.cols} {w.dtype} x ~ N(0, {w.std:g}^2), scale {w.scale:g}; "
                        f"y same dtype + fp32 LSE",
            "rows": w.rows, "cols": w.cols, "element": w.dtype,
            "compulsory_hbm_bytes": nbytes,
            "kernel_ms": kernel_ms,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": measured_traffic(w.name, SOFTMAX_SOURCE),
        },
    }
    out["provenance"] = provenance(w.seed)
    out["cpu_baseline"] = None if args.no_cpu_baseline else softmax_cpu_baseline(w, x, args.cpu_rows_softmax)
    out["config"].update(event_stats(starts, ends))
    print(json.dumps(out), flush=True)


def bwd_flops(w) -> float:
    """Five products per (query, visible key) pair -- S = Q K^T recomputed, dP = dO V^T,
    dV = P^T dO, dQ = dS K, dK = dS^T Q -- at 2 d FLOPs each: 2.5 times the forward's count
    (same causal halving)."""
    return 2.5 * flops(w)


def bwd_bytes(w) -> int:
    """Compulsory bytes: bf16 Q, K, V, dO and fp32 O, LSE read once; fp32 dQ, dK, dV written."""
    n = w.B * w.H * w.N
    return 4 * 2 * n * w.d + 4 * n * w.d + 4 * n + 3 * 4 * n * w.d


def bench_backward(args):
    import torch

    from io_aware_softmax_mifa_amd import binding
    from io_aware_softmax_mifa_amd import workloads as W

    w = W.by_name(args.workload[: -len("-bwd")])
    scale = W.fp32_scale(w.d)
    log(f"backward of workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} dist={w.dist}")
    q, k, v = W.make_workload_inputs(w)
    do = W.make_grad_output(w.B, w.H, w.N, w.d, w.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gq, gk, gv, gdo = (t.to(dev) for t in (q, k, v, do))
    o, lse = binding.attention(gq, gk, gv, causal=w.causal, scale=scale)
    dq = torch.empty(w.shape, dtype=torch.float32, device=dev)
    dk, dv = torch.empty_like(dq), torch.empty_like(dq)
    need = binding.mifa_bwd_workspace_bytes(w.B, w.H, w.N)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        st = binding.mifa_bwd_raw(gq, gk, gv, o, lse, gdo, dq, dk, dv, w.B, w.H, w.N, w.N, w.d, w.causal, scale,
                                  ws, ws.numel(), stream.cuda_stream)
        if st != 0:
            raise binding.MifaError(st, binding.mifa_status_string(st))

    args.warmup = warm_up(step, args.warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    call_ms = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {call_ms:.4f} ms/call (HIP events; "
        "row_dot + dq + dkdv kernels)")
    if args.copy_calibration:
        copy_calibration(dev)
    f = bwd_flops(w)
    value = f / (ms_per_step * 1e-3) / 1e12
    achieved = f / (call_ms * 1e-3) / 1e12
    out = {
        "metric": "attention bwd TFLOP/s (bf16, 2.5x forward FLOP convention) and % of MI355X bf16 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. bf16 Q/K/V/dO)",
        "config": {
            "workload": f"{w.name} backward: B={w.B} H={w.H} N={w.N} d={w.d} causal={int(w.causal)} bf16 Q,K,V,dO "
                        f"~ N(0,1); fp32 O + LSE from the forward; fp32 dQ, dK, dV",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": bool(w.causal),
            "flop_per_step": f,
            "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
            "call_ms": call_ms,
            "compulsory_hbm_bytes": bwd_bytes(w),
            "workspace_bytes": need,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(args.workload, BWD_SOURCE),
            "kernels": "row_dot + dq + dkdv (one mifa_bwd call)",
        },
    }
    out["clock"] = sample_clock(step, value)
    out["provenance"] = provenance(w.seed)
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        from oracle import attention_bwd_fp64

        heads, L = min(16, w.H), min(8192, w.N)
        sub = [t[:1, :heads, :L].contiguous() for t in (q, k, v, do)]
        t0 = time.perf_counter()
        attention_bwd_fp64(*sub, causal=w.causal, scale=scale)
        dt = time.perf_counter() - t0
        pairs = L * L / 2 if w.causal else L * L
        sample_f = heads * 10.0 * pairs * w.d
        out["cpu_baseline"] = {
            "value": sample_f / dt / 1e12,
            "unit": "TFLOP/s",
            "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"{heads} heads of batch 0, first {L} positions each (a causal prefix is a complete "
                       f"smaller problem), float64 NumPy oracle with the full P materialised, {dt:.2f} s; "
                       f"credited with the same 10 d FLOPs per visible pair"),
            "seconds": dt,
            **host_info(),
        }
    out["config"].update(event_stats(starts, ends))
    print(json.dumps(out), flush=True)


def bench_gemm_reference(args):
    """Context leg, not this library's code: the vendor library's dense bf16 GEMM
    (`torch.matmul`, hipBLASLt on ROCm) at M = N = K = 8192 with its sustained clock, i.e. what a
    plain contraction with no softmax between its products reaches on this GPU.  The attention
    legs' fractions of the 2.5 PFLOP/s peak read against it."""
    import torch

    M = N = K = 8192
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator().manual_seed(11)
    a = torch.randn(M, K, generator=g).to(dev, torch.bfloat16)
    b = torch.randn(K, N, generator=g).to(dev, torch.bfloat16)
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        torch.matmul(a, b, out=c)

    args.warmup = warm_up(step, args.warmup)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    call_ms = sum(x.elapsed_time(y) for x, y in zip(starts, ends)) / args.steps
    f = 2.0 * M * N * K
    value = f / (ms_per_step * 1e-3) / 1e12
    achieved = f / (call_ms * 1e-3) / 1e12
    log(f"timed {args.steps} GEMMs: {ms_per_step:.4f} ms/step wall, {call_ms:.4f} ms/call (HIP events)")
    out = {
        "metric": "bf16 GEMM TFLOP/s (torch.matmul, vendor library; reference, not mifa) and % of MI355X bf16 "
                  "MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 matrices)",
        "config": {"workload": f"GEMM-ref: C = A B, M=N=K={M}, bf16 in and out, fp32 accumulation (hipBLASLt)",
                   "M": M, "N": N, "K": K, "flop_per_step": f, "call_ms": call_ms,
                   "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "cpu_baseline": None,
    }
    out["clock"] = sample_clock(step, value)
    out["provenance"] = provenance(11)
    out["config"].update(event_stats(starts, ends))
    print(json.dumps(out), flush=True)


def bench_hbm_reference(args):
    """Context leg, not this library's code: the vendor's plain streaming kernels on this GPU's
    HBM, what the HBM-bound legs (split-KV decode, row softmax) read against.  One step = a 1 GiB
    device copy (`copy_`, the runtime's copy kernel: 1 GiB read and 1 GiB written); `value` is its
    rate.  Timed separately after it: a 2 GiB bf16 tensor summed (`torch.sum`, read once, fp32
    accumulation), whose read rate goes into `config`."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1)
    b = torch.empty_like(a)

    def step():
        b.copy_(a)

    def timed(fn, steps):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return wall, sum(x.elapsed_time(y) for x, y in zip(starts, ends)) / steps, starts, ends

    args.warmup = warm_up(step, args.warmup)
    ms_per_step, call_ms, starts, ends = timed(step, args.steps)
    nbytes = 2 * 2 * a.numel()
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    del a, b
    x = torch.empty(1 << 30, dtype=torch.bfloat16, device=dev).fill_(0.5)
    out = torch.empty((), dtype=torch.float32, device=dev)

    def total():
        torch.sum(x, dim=0, dtype=torch.float32, out=out)

    for _ in range(5):
        total()
    _, sum_ms, _, _ = timed(total, args.steps)
    sum_gbs = 2 * x.numel() / (sum_ms * 1e-3) / 1e9
    log(f"timed {args.steps} copies of 2 x {nbytes // 2} bytes: {ms_per_step:.4f} ms/step wall, {call_ms:.4f} "
        f"ms/call; sum of {2 * x.numel()} bytes: {sum_ms:.4f} ms/call")
    out_line = {
        "metric": "HBM GB/s of a device copy (copy_, vendor runtime; reference, not mifa) and % of MI355X HBM "
                  "bandwidth",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (constant-filled tensors)",
        "config": {"workload": f"HBM-ref: copy of {nbytes // 2} bytes (read and written once); then a sum of "
                               f"{2 * x.numel()} bytes of bf16 (read once)",
                   "bytes_per_step": nbytes, "call_ms": call_ms, "pct_of_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
                   "sum_ms": sum_ms, "sum_gbs": sum_gbs, "sum_pct_of_hbm_peak": 100.0 * sum_gbs / PEAK_HBM_GBS},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": None},
        "cpu_baseline": None,
    }
    out_line["provenance"] = provenance(0)
    out_line["config"].update(event_stats(starts, ends))
    print(json.dumps(out_line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up launches (default: at least 30 and at least 0.5 s of them)")
    ap.add_argument("--workload", default="C4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=131072)
    ap.add_argument("--cpu-rows-softmax", type=int, default=0, help="0: every row")
    ap.add_argument("--cold", action="store_true",
                    help="forward legs: rotate through input/output copies larger than twice the LLC")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the kernel has no "
              "multi-GPU path: heads shard across GPUs with no communication, so the per-GPU figure is the "
              "one-GPU run on that GPU's share).", file=sys.stderr)
        sys.exit(2)

    if args.workload == "GEMM-ref":
        return bench_gemm_reference(args)
    if args.workload == "HBM-ref":
        return bench_hbm_reference(args)
    if args.workload.startswith("SM"):
        return bench_softmax(args)
    if args.workload.startswith("D"):
        return bench_decode(args)
    if args.workload.endswith("-bwd"):
        return bench_backward(args)

    import torch

    from io_aware_softmax_mifa_amd import binding
    from io_aware_softmax_mifa_amd import workloads as W

    w = W.by_name(args.workload)
    scale = W.fp32_scale(w.d)
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} dist={w.dist}")
    q, k, v = W.make_workload_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = compulsory_bytes(w)
    # --cold: rotate through enough copies of the inputs and outputs that the working set is
    # more than twice the 256 MiB last-level cache, so every step's bytes come from HBM.
    copies = (2 * LLC_BYTES) // cb + 2 if args.cold else 1
    bufs = []
    for _ in range(copies):
        bufs.append((*(t.to(dev) for t in (q, k, v)), torch.empty(w.shape, dtype=torch.float32, device=dev),
                     torch.empty(w.shape[:3], dtype=torch.float32, device=dev)))
    o, lse = bufs[0][3], bufs[0][4]
    stream = torch.cuda.current_stream(dev)
    turn = [0]

    def step():
        dq, dk, dv, oo, ll = bufs[turn[0] % copies]
        turn[0] += 1
        binding.mifa_fwd(dq, dk, dv, oo, ll, w.B, w.H, w.N, w.d, w.causal, scale, stream.cuda_stream)

    args.warmup = warm_up(step, args.warmup)
    log(f"warmup {args.warmup} done" + (f" ({copies} rotating copies, {copies * cb / 2**20:.0f} MiB)" if args.cold else ""))

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step wall, {kernel_ms:.4f} ms/launch (HIP events)")
    # outputs of the last timed launch, for its parity against the oracle rows of the CPU baseline
    last_o, last_lse = bufs[(turn[0] - 1) % copies][3].cpu(), bufs[(turn[0] - 1) % copies][4].cpu()

    f = flops(w)
    value = f / (ms_per_step * 1e-3) / 1e12
    gbs = cb / (kernel_ms * 1e-3) / 1e9

    if args.copy_calibration:
        copy_calibration(dev)

    out = {
        "metric": (f"attention fwd TFLOP/s (bf16, {'causal' if w.causal else 'non-causal'}) and % of MI355X bf16 "
                   "MFMA peak"),
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. bf16 Q/K/V)",
        "config": {
            "workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={int(w.causal)} "
                        f"bf16 Q,K,V ~ {'N(0,1)' if w.dist == 'normal' else 'stress'}; fp32 O + LSE",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": bool(w.causal),
            "flop_per_step": f,
            "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
            "kernel_ms": kernel_ms,
            "compulsory_hbm_bytes": cb,
            "compulsory_gbs": gbs,
            "flop_per_byte": f / cb,
            "cold_cache": bool(args.cold),
            "rotating_copies": copies,
        },
        "roofline": forward_roofline(f, cb, kernel_ms),
    }
    out["roofline"]["traffic"] = measured_traffic(w.name + ("-cold" if args.cold else ""))
    out["clock"] = sample_clock(step, value)
    if out["clock"].get("pct_of_clock_adjusted_peak") is not None:
        log(f"sustained clock {out['clock']['median_mhz']:.0f} MHz: {out['clock']['pct_of_clock_adjusted_peak']:.1f}% of "
            "the peak at that clock")
    out["provenance"] = provenance(w.seed)
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_rows} sampled rows")
        out["cpu_baseline"], out["parity"] = cpu_baseline(w, q, k, v, scale, args.cpu_rows, last_o, last_lse)
        log(f"parity of the last timed launch on {out['parity']['rows']} rows: O max {out['parity']['o_max_abs']:.3e} "
            f"mean {out['parity']['o_mean_abs']:.3e}, LSE max {out['parity']['lse_max_abs']:.3e}")
    else:
        out["cpu_baseline"], out["parity"] = None, None
    out["config"].update(event_stats(starts, ends))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
