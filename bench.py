"""Benchmark of the attention forward (and backward) pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd]

A step is one fa2_fwd call over one batch of the workload (all of its heads
and query rows), inputs already resident in HBM.  Before the W counted
warm-up steps, untimed steps run back to back for --prewarm seconds (0.3 by
default) so that short kernels are not timed while the clock ramps up.  The default workload is the
fp32 shape the CUDA project page benchmarks (B=4, H=12, M=N=2048, D=64,
non-causal).  Prints ONE JSON line with the whole-job throughput
(4*B*H*M*N*D flop per step, halved for causal) and:

* roofline: the kernel's achieved TFLOP/s = counted flop per launch / mean
  launch duration (HIP events on the launch stream over the timed region),
  against MI355X's dense MFMA peak for the dtype; traffic = HBM bytes per
  launch from the committed rocprofv3 counter summary, when it was taken on
  the current kernel source;
* sclk: the shader clock the amdgpu kernel driver reports (sysfs) while the timed steps run;
* cpu_baseline: the CPU oracle timed on this host on the same workload
  (value), and on each of the five configurations with the max-abs error of
  the GPU's O and L against it (configs; the long-context one on its sample
  of query rows, with the full run extrapolated and labelled as such), plus
  the tiny configuration on a single core;
* workloads: per-launch latency (median of 100 after 25 warm-ups, with and
  without an L2/MALL flush before each launch) of every workload;
* backward: per-call latency of fa2_bwd (its dQ, dK/dV and, for fp32, Delta kernels) on the
  workloads of workloads.BACKWARD, counted as 10*B*H*M*N*D flop (halved for
  causal).

With --pass bwd the timed step is one fa2_bwd call instead (the forward's o
and lse are computed once beforehand), counted the same way.
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
sys.path.insert(0, ROOT)

METRIC = ("attention fwd TFLOP/s (4·B·H·M·N·D) and % of MFMA peak; "
          "latency µs, 1 MI355X")
METRIC_BWD = ("attention bwd TFLOP/s (10·B·H·M·N·D) and % of MFMA peak; "
              "latency µs, 1 MI355X")
# MI355X dense matrix peaks (AMD's published figures): bf16 2.5 PFLOP/s
# (256 CU x 2.4 GHz x 4096 flop/clk), fp32 157.3 TFLOP/s.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
# Context only: the CUDA project page's hand-written fp32 kernel on an RTX 4080
# at B=4,H=12,M=N=2048,D=64 took 3810.30 us, i.e. 13.53 TFLOP/s by this count.
PAGE_REFERENCE_US = {"mha_f32_2k": 3810.30}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the forward kernels and the helpers they include
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_23_amd", "csrc", name)
               for name in ("fa2_fwd.hip", "fa2_common.h")]


def kernel_source_hash() -> str:
    """sha256 of the forward kernel sources with comments and blank space
    removed, so that counters stay attached to the code they were taken on."""
    import re
    src = ""
    for path in KERNEL_SRCS:
        with open(path) as f:
            src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())
    return hashlib.sha256(src.encode()).hexdigest()


def load_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the kernel source that is built now."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get("workloads", {}).get(workload)
    if not entry or data.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def dominant_kernel(w, splits: int = 1) -> str:
    """The forward kernel the library launches for this workload (its
    dispatch table: fp32 kernel, or the 16-bit kernel, ping-pong on the
    dense unwindowed path unless a head has at most 64 rows),
    followed by the combine kernel when the key range is split."""
    # rows per head of the kernel view: the grouped query heads of a K/V head
    # form one row sequence when there is no mask
    rows = w.M * (w.H // w.kv_heads) if not w.causal and w.window == (-1, -1) else w.M
    if w.dtype == "f32":
        k = "fa2_fwd_f32_kernel"
    elif w.lengths is not None or w.window != (-1, -1) or rows <= 64:
        k = "fa2_fwd_half_kernel"
    else:
        k = "fa2_fwd_half_pp_kernel"
    return k + (f" x{splits} splits + fa2_merge_kernel" if splits > 1 else "")


def roofline_of(w, seconds: float):
    """(bound, achieved, peak, unit): MFMA-bound when the workload's counted
    flop per algorithmic byte exceeds the ridge point of its dtype, else
    HBM-bound (decode-like shapes)."""
    peak = PEAK_TFLOPS[w.dtype]
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    if w.flops / w.compulsory_bytes >= ridge:
        return "mfma", w.flops / seconds / 1e12, peak, "TFLOP/s"
    return "hbm", w.compulsory_bytes / seconds / 1e9, HBM_PEAK_GBS, "GB/s"


def prewarm(fn, seconds: float):
    """Run the step back to back for `seconds` of wall time before any
    counted warm-up, so that short kernels are timed at the clock a busy GPU
    settles at rather than while the clock is still ramping up from idle."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(fn, stream, warmup: int, reps: int, flush=None, prewarm_s: float = 0.0):
    """Per-launch durations (ms) from HIP events recorded on the launch stream."""
    import torch
    if prewarm_s > 0:
        prewarm(fn, prewarm_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        times.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in times]


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


# parity tolerances of the comparison with the oracle (max-abs on O, on L)
TOLERANCE = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-3), "f16": (5e-3, 1e-3)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _f32_carrier(t):
    """The exact float32 values of an input tensor (bf16 / fp16 widened)."""
    import torch
    return t.to(torch.float32).contiguous().numpy()


def _sampled_flops(w, rows) -> float:
    """Counted work of the listed query rows: 4*D flop per visible (query,
    key) pair, over every head."""
    if rows is None:
        return w.flops
    pairs = sum(min(int(i) + 1, w.N) if w.causal else w.N for i in rows)
    return 4.0 * w.B * w.H * w.D * pairs


def cpu_baseline(headline, gpu_forward):
    """The fp64 oracle, as it stands, on this host: every workload of the
    five configurations (all threads; config 4 on its seeded sample of query
    rows, with the full run extrapolated by visible pairs and labelled as
    such), the tiny configuration once more on one core, and the max-abs
    error of the GPU result against it per configuration.  `gpu_forward(w, q,
    k, v)` returns the GPU's (o, lse) as float64 arrays."""
    import numpy as np
    import oracle
    import workloads
    threads = oracle.max_threads()
    configs = []
    head = None
    for name in workloads.ORDER:
        w = workloads.get(name)
        q, k, v = workloads.workload_inputs(w)
        rows = workloads.sample_rows(w)
        rows_np = None if rows is None else rows.numpy()
        qa, ka, va = _f32_carrier(q), _f32_carrier(k), _f32_carrier(v)
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention(qa, ka, va, w.scale, w.causal, rows=rows_np)
        dt = time.perf_counter() - t0
        del qa, ka, va
        o_gpu, l_gpu = gpu_forward(w, q, k, v)
        if rows_np is not None:
            o_gpu, l_gpu = o_gpu[:, :, rows_np], l_gpu[:, :, rows_np]
        err_o = float(np.abs(o_gpu - o_ref).max())
        err_l = float(np.abs(l_gpu - l_ref).max())
        tol_o, tol_l = TOLERANCE[w.dtype]
        flops = _sampled_flops(w, rows_np)
        entry = {"workload": w.name, "rows_checked": "all" if rows_np is None else
                 f"{len(rows_np)} per head (seeded sample, rows 0 and M-1 included)",
                 "oracle_s": round(dt, 3), "oracle_tflops": round(flops / dt / 1e12, 4), "cores": threads,
                 "max_abs_o": err_o, "max_abs_l": err_l, "tolerance_o": tol_o, "tolerance_l": tol_l,
                 "within_tolerance": bool(err_o <= tol_o and err_l <= tol_l)}
        if rows_np is not None:
            entry["oracle_s_full_extrapolated"] = round(dt * w.flops / flops, 1)
            entry["extrapolation"] = "measured time x (visible pairs of every row / of the sampled rows)"
        configs.append(entry)
        if w.name == headline.name:
            head = (flops / dt / 1e12, dt, rows_np)
        del q, k, v, o_ref, l_ref, o_gpu, l_gpu
    # the tiny configuration on one core
    w1 = workloads.get(workloads.ORDER[0])
    q, k, v = (_f32_carrier(t) for t in workloads.workload_inputs(w1))
    t0 = time.perf_counter()
    oracle.attention(q, k, v, w1.scale, w1.causal, threads=1)
    single = time.perf_counter() - t0
    value, seconds, rows_np = head
    sample = (f"all {headline.B}x{headline.H}x{headline.M} query rows of {headline.name}, one pass"
              if rows_np is None else f"{len(rows_np)} sampled rows per head of {headline.name}")
    return {"value": value, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "sample": sample,
            "seconds": seconds, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_core": {"workload": w1.name, "seconds": round(single, 4),
                            "tflops": round(w1.flops / single / 1e12, 5), "cores": 1},
            "configs": configs}


class SclkSampler:
    """Shader clock while the GPU works: the current-clock line of the amdgpu
    driver's pp_dpm_sclk table, read every few milliseconds by a thread;
    None where the file is not readable."""
    PATHS = ("/sys/class/drm/card0/device/pp_dpm_sclk",)

    def __init__(self, period_s: float = 0.002):
        import threading
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self.path = next((p for p in self.PATHS if os.access(p, os.R_OK)), None)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    mhz = line.split(":", 1)[1].strip().rstrip("*").strip()
                    return float(mhz.lower().replace("mhz", ""))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                x = self._read()
            except (OSError, ValueError):
                x = None
            if x is not None:
                self.samples.append(x)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path is not None:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        return {"median_mhz": median(self.samples), "min_mhz": min(self.samples), "max_mhz": max(self.samples),
                "samples": len(self.samples), "source": self.path}


COPY_BYTES = 256 * 1024 * 1024


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, five times: under
    rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch give the counter
    reading for a known number of HBM bytes read and written."""
    import torch
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "dispatches": 5}), flush=True)
    return 0


def _read_counter_csv(path, counter):
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload, out=TRAFFIC_FILE):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch)
    into HBM bytes per launch of the attention kernel, each counter scaled by
    its reading for the plain copy of COPY_BYTES (copy_calibration)."""
    def med_for(rows, pred):
        vals = [v for name, v in rows if pred(name)]
        if not vals:
            raise ValueError("no matching dispatches")
        return median(vals), len(vals)

    is_fa2 = lambda n: "fa2_fwd_" in n
    is_copy = lambda n: "copyBuffer" in n or "copy" in n.lower()
    cf, _ = med_for(_read_counter_csv(copy_fetch_csv, "FETCH_SIZE"), is_copy)
    cw, _ = med_for(_read_counter_csv(copy_write_csv, "WRITE_SIZE"), is_copy)
    f, nf = med_for(_read_counter_csv(fetch_csv, "FETCH_SIZE"), is_fa2)
    wr, nw = med_for(_read_counter_csv(write_csv, "WRITE_SIZE"), is_fa2)
    fetch_scale = COPY_BYTES / (cf * 1024.0)
    write_scale = COPY_BYTES / (cw * 1024.0)
    entry = {"fetch_bytes": f * 1024.0 * fetch_scale, "write_bytes": wr * 1024.0 * write_scale,
             "fetch_kib_raw": f, "write_kib_raw": wr, "fetch_scale": fetch_scale,
             "write_scale": write_scale, "dispatches": [nf, nw]}
    entry["bytes_per_launch"] = entry["fetch_bytes"] + entry["write_bytes"]
    try:
        with open(out) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    if data.get("kernel_source_sha256") != kernel_source_hash():
        data = {"kernel_source_sha256": kernel_source_hash(), "workloads": {}}
    data["workloads"][workload] = entry
    with open(out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({workload: entry}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--workload", default="mha_f32_2k")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward pass (fa2_bwd)")
    ap.add_argument("--prewarm", type=float, default=0.3,
                    help="seconds of back-to-back untimed steps before the warm-up steps (clock settling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="skip the per-workload table")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (calibrates HBM counters)")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json for --workload from rocprofv3 counter CSVs")
    args = ap.parse_args(argv)

    if args.copy_calibration:
        return copy_calibration()
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, workload=args.workload)

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the forward pass shards over batch*head with no exchange, "
                                   "but multi-GPU runs are not part of it)"}), flush=True)
        return 2

    import torch
    import exact_attention_23_amd as fa2
    import workloads

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def code_of(w):
        return {"f32": fa2.FA2_DTYPE_F32, "bf16": fa2.FA2_DTYPE_BF16, "f16": fa2.FA2_DTYPE_F16}[w.dtype]

    def splits_of(w):
        if w.n_splits != 0:
            return w.n_splits
        return fa2.fa2_fwd_num_splits(w.B, w.H, w.kv_heads, w.M, w.N, w.D, int(w.causal), code_of(w))

    def setup(w):
        q, k, v = (t.to(dev) for t in workloads.workload_inputs(w))
        o = torch.empty_like(q)
        if w.lengths is not None:
            # packed sequences: lse [H, total]; the "workspace" slot carries the offsets
            lse = torch.empty((w.H, q.shape[1]), dtype=torch.float32, device=dev)
            return q, k, v, o, lse, workloads.cu_seqlens(w).to(dev), 1
        lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev)
        splits = splits_of(w)
        need = fa2.fa2_fwd_workspace_bytes(w.B, w.H, w.M, w.D, splits)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        return q, k, v, o, lse, ws, splits

    def launcher(w, bufs):
        q, k, v, o, lse, ws, splits = bufs
        code = code_of(w)
        if w.lengths is not None:
            total = q.shape[1]
            args_ = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                     ws.data_ptr(), w.B, w.H, w.kv_heads, total, total, max(w.lengths), w.D, w.scale,
                     int(w.causal), w.window[0], w.window[1], code, stream.cuda_stream)
            call = fa2.fa2_fwd_varlen
        elif w.window != (-1, -1):
            args_ = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.kv_heads, w.M, w.N, w.D, w.scale, int(w.causal), w.window[0], w.window[1],
                     code, stream.cuda_stream)
            call = fa2.fa2_fwd_local
        elif w.Hk is None and splits == 1:
            # the plain entry point
            args_ = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.M, w.N, w.D, w.scale, int(w.causal), code, stream.cuda_stream)
            call = fa2.fa2_fwd
        else:
            args_ = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                     w.B, w.H, w.kv_heads, w.M, w.N, w.D, w.scale, int(w.causal), code, splits,
                     ws.data_ptr(), ws.numel(), stream.cuda_stream)
            call = fa2.fa2_fwd_ex

        def fn():
            st = call(*args_)
            if st != fa2.FA2_OK:
                raise fa2.Fa2Error(st)
        return fn

    def bwd_setup(w):
        q, k, v, o, lse, ws, splits = setup(w)
        launcher(w, (q, k, v, o, lse, ws, splits))()  # the forward's o and lse
        do = workloads.make_dout(w.B, w.H, w.M, w.D, w.dtype, w.seed).to(dev)
        delta = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        del ws
        return q, k, v, o, lse, do, torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), delta

    def bwd_launcher(w, b):
        args_ = tuple(t.data_ptr() for t in b) + (w.B, w.H, w.kv_heads, w.M, w.N, w.D, w.scale,
                                                   int(w.causal), code_of(w), stream.cuda_stream)

        def fn():
            st = fa2.fa2_bwd(*args_)
            if st != fa2.FA2_OK:
                raise fa2.Fa2Error(st)
        return fn

    w = workloads.get(args.workload)
    backward = args.which == "bwd"
    if backward:
        bufs = bwd_setup(w)
        fn = bwd_launcher(w, bufs)
        step_flops = w.bwd_flops
    else:
        bufs = setup(w)
        fn = launcher(w, bufs)
        step_flops = w.flops

    # ---- the timed steps: W untimed, then exactly K, synchronised on both sides
    # (preceded by --prewarm seconds of untimed steps that let the clock settle)
    if args.prewarm > 0:
        prewarm(fn, args.prewarm)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    events = []
    with SclkSampler() as sclk:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            events.append((s, e))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in events]
    ms_per_step = wall * 1e3 / args.steps
    mean_launch_ms = sum(launch_ms) / len(launch_ms)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    if backward:
        # one fa2_bwd call on one stream: 16-bit dQ (with Delta) then dK/dV;
        # fp32 Delta, dK/dV, dQ
        peak = PEAK_TFLOPS[w.dtype]
        achieved = step_flops / (mean_launch_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": None,
                    "mean_launch_us": round(mean_launch_ms * 1e3, 2),
                    "kernel": ("fa2_bwd: fa2_bwd_delta_f32_kernel + fa2_bwd_dkdv_f32_kernel + fa2_bwd_dq_f32_kernel"
                               if w.dtype == "f32" else
                               "fa2_bwd: fa2_bwd_dq_kernel (with Delta) + "
                               + ("fa2_bwd_dkdv_pair_kernel" if w.D == 128 else "fa2_bwd_dkdv_kernel"))
                              + f" (D={w.D}, causal={int(w.causal)})"}
        splits = 1
    else:
        bound, achieved, peak, unit = roofline_of(w, mean_launch_ms * 1e-3)
        roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                    "frac": round(achieved / peak, 4), "traffic": load_traffic(w.name),
                    "mean_launch_us": round(mean_launch_ms * 1e3, 2),
                    "kernel": f"{dominant_kernel(w, bufs[6])} (D={w.D}, causal={int(w.causal)})"}
        splits = bufs[6]

    ref_us = None if backward else PAGE_REFERENCE_US.get(w.name)
    vs_baseline = None if ref_us is None else round(value / (w.flops / (ref_us * 1e-6) / 1e12), 3)

    result = {
        "metric": METRIC_BWD if backward else METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": vs_baseline,
        "dtype": w.dtype, "data": "synthetic (seeded Gaussian Q/K/V)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hk": w.kv_heads, "M": w.M, "N": w.N,
                   "D": w.D, "causal": w.causal, "io_dtype": w.dtype, "kv_splits": splits,
                   "pass": args.which,
                   "global_batch": w.B, "seq_len": w.M, "parallelism": "single GPU"},
        "roofline": roofline,
        "sclk": sclk.summary(),
    }
    del bufs

    # ---- per-workload latency table (each launch timed alone)
    if not args.no_extras:
        flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
        table = {}
        for name in workloads.ORDER + workloads.WIDENED:
            wx = workloads.get(name)
            bx = setup(wx)
            fx = launcher(wx, bx)
            with SclkSampler() as sc:
                hot = time_launches(fx, stream, 25, 100, prewarm_s=args.prewarm)
            cold = time_launches(fx, stream, 3, 20, flush=flush_buf.zero_)
            us, us_cold = median(hot) * 1e3, median(cold) * 1e3
            tf = wx.flops / (us * 1e-6) / 1e12
            bound, ach, pk, unit = roofline_of(wx, us * 1e-6)
            shape = f"B={wx.B},H={wx.H},Hk={wx.kv_heads},M={wx.M},N={wx.N},D={wx.D}"
            if wx.window != (-1, -1):
                shape += f",window={wx.window}"
            if wx.lengths is not None:
                shape += f",packed lengths={list(wx.lengths)}"
            table[name] = {"shape": shape,
                           "dtype": wx.dtype, "causal": wx.causal, "kv_splits": bx[6],
                           "us_median": round(us, 2), "us_median_l2_flushed": round(us_cold, 2),
                           "tflops": round(tf, 2), "frac_of_mfma_peak": round(tf / PEAK_TFLOPS[wx.dtype], 4),
                           "hbm_gbs_compulsory": round(wx.compulsory_bytes / (us * 1e-6) / 1e9, 1),
                           "bound": bound, "frac_of_bound": round(ach / pk, 4),
                           "sclk_mhz_median": (sc.summary() or {}).get("median_mhz")}
            # the dtype's dense peak scaled to the clock the launches ran at
            # (AMD's peak figures assume 2.4 GHz)
            mhz = table[name]["sclk_mhz_median"]
            table[name]["frac_of_mfma_peak_at_sclk"] = (
                round(tf / (PEAK_TFLOPS[wx.dtype] * mhz / 2400.0), 4) if mhz else None)
            del bx, fx
        result["workloads"] = table
        # backward passes (one fa2_bwd call each)
        btable = {}
        for name in workloads.BACKWARD:
            wx = workloads.get(name)
            bx = bwd_setup(wx)
            fx = bwd_launcher(wx, bx)
            hot = time_launches(fx, stream, 10, 50, prewarm_s=args.prewarm)
            cold = time_launches(fx, stream, 3, 10, flush=flush_buf.zero_)
            us, us_cold = median(hot) * 1e3, median(cold) * 1e3
            tf = wx.bwd_flops / (us * 1e-6) / 1e12
            btable[name] = {"shape": f"B={wx.B},H={wx.H},Hk={wx.kv_heads},M={wx.M},N={wx.N},D={wx.D}",
                            "dtype": wx.dtype, "causal": wx.causal, "us_median": round(us, 2),
                            "us_median_l2_flushed": round(us_cold, 2), "tflops": round(tf, 2),
                            "frac_of_mfma_peak": round(tf / PEAK_TFLOPS[wx.dtype], 4), "bound": "mfma"}
            del bx, fx
        del flush_buf
        result["backward"] = btable

    if not args.no_cpu and not backward:
        import numpy as np

        def gpu_forward(wx, q, k, v):
            o, lse = fa2.forward(q.to(dev), k.to(dev), v.to(dev), causal=wx.causal)
            torch.cuda.synchronize()
            return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(w, gpu_forward)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
