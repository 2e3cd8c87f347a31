#!/usr/bin/env python3
"""Attention throughput on one MI355X: forward + recompute backward.

One step is the whole hot path once over one batch of seeded synthetic input:
attn_fwd, then the backward's two stages (attn_bwd_dq_stats, the dQ stage
that also writes the row statistics, then attn_bwd_dkdv: exactly what
attn_bwd launches), all through the C ABI on one stream.  The
workload is the causal forward + backward problem B=8, H=16, N=2048, d=64
(bf16 I/O, fp32 accumulation).  Inputs are resident in device memory before
the timed region starts.

FLOP convention (algorithmic): forward 4*B*H*N^2*d, backward 10*B*H*N^2*d
(the five products S, dV, dP, dK, dQ), both halved for a causal mask.  The
backward's recomputation of S and dP inside the dQ kernel is executed but not
counted.

Printed: one JSON line with the step throughput, the roofline of the dominant
kernel (durations from HIP events on the launch stream), every kernel's
duration, a forward sweep over the other workloads, the split-K/V forward on
the key/value-cache workloads (decode, append; GB/s against HBM), the
block-sparse forward on a local + global + random block mask (TFLOP/s over
the visible pairs, and the dense forward of the same shape beside it), the
packed variable-length forward and backward on a document batch (and the
same documents padded to the longest), and the fp64 CPU oracle timed on a bounded sample of
the same workload.  A backward sweep times attn_bwd alone (algorithmic
10*B*H*N^2*d, halved for causal) on d = 128 and 256 shapes, one of them a
grouped-query shape short enough that the dK/dV stage splits its query heads.
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

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # dense bf16 MFMA: CUs x FLOP/clk/CU x clock
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd(+bwd) TFLOP/s on 1 MI355X; % of peak bf16 MFMA"
CSRC = os.path.join(ROOT, "exact_attention_87_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def warm_up(fn, min_calls: int, min_ms: float = 60.0):
    """Untimed calls of fn: at least min_calls, and until the GPU has been kept
    busy for min_ms.  Its clocks ramp up from idle over tens of milliseconds
    (measured: the B=8 H=16 N=2048 d=64 step takes 0.40 ms after 5 warm-up
    steps and a steady 0.34 ms after 50-200), and host work between the sweep
    cases lets them fall again."""
    import torch

    t0 = time.perf_counter()
    for _ in range(min_calls):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank lines removed, so a
    comment edit does not invalidate counters taken on the same code."""
    import re

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name == "attn_clock.hip":  # the clock probe: no attention kernel
            continue
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(name.encode())
        h.update(code.encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


# Counter runs read by --traffic-from: run name -> this script's arguments.  Each run
# is profiled three times, all with --copy-mib 512 (the calibration copy):
#   rocprofv3 --pmc FETCH_SIZE -d DIR/<run>_FETCH_SIZE -o run --output-format csv
#       -- python3 bench.py <args> --steps 2 --warmup 1 --copy-mib 512
#   the same with WRITE_SIZE into DIR/<run>_WRITE_SIZE, and
#   rocprofv3 --kernel-trace --stats -d DIR/<run>_trace -o run --output-format csv
#       -- python3 bench.py <args> --steps 30
TRAFFIC_RUNS = {
    "step": "--no-sweep --cpu-seconds 0",
    "fwd2": "--fwd-only 2", "fwd3": "--fwd-only 3", "fwd4": "--fwd-only 4",
    "bwd4": "--bwd-only 4",
    "decode": "--splitkv-only decode",
    "sparse": "--sparse-only local_global",
    "varlen": "--varlen-only docs",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
CALIBRATION_KIB = 512 * 1024.0  # the copy reads and writes 512 MiB


def kernel_label(mangled: str) -> str:
    """Readable name of one of this library's kernels: the name and its template
    arguments (element type, head dimension, flags)."""
    import re

    if mangled.startswith("attn::"):
        return mangled.split("(")[0][len("attn::"):]
    m = re.match(r"_ZN4attn\d+(\w+?)I(.*?)EEv", mangled)
    if m is None:
        return mangled
    args = []
    for t in re.finditer(r"DF16b|DF16_|Li(\d+)E|Lb([01])E", m.group(2)):
        if t.group(0) == "DF16b":
            args.append("__bf16")
        elif t.group(0) == "DF16_":
            args.append("_Float16")
        elif t.group(1) is not None:
            args.append(t.group(1))
        else:
            args.append("true" if t.group(2) == "1" else "false")
    return m.group(1) + "<" + ", ".join(args) + ">"


def counter_run(indir: str, run: str, timed: int = 30):
    """Per-kernel HBM bytes per launch of one profiled run: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, averaged over the dispatches) scaled so the
    calibration copy reads 512 MiB each, and the average duration of each
    kernel's last `timed` traced dispatches (the timed launches)."""
    import collections
    import csv

    def per_kernel(ctr):
        agg = collections.defaultdict(list)
        with open(os.path.join(indir, f"{run}_{ctr}", "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        if COPY_KERNEL not in agg:
            raise SystemExit(f"traffic: no calibration copy in {run}_{ctr} "
                             "(profile the run with --copy-mib 512)")
        res = {k: sum(v) / len(v) for k, v in agg.items()}
        # the calibration copy is the run's largest copy (a run may hold smaller ones)
        res[COPY_KERNEL] = max(agg[COPY_KERNEL])
        return res

    spans = collections.defaultdict(list)
    with open(os.path.join(indir, f"{run}_trace", "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            spans[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    avg_us = {}
    for k, v in spans.items():
        last = sorted(v)[-timed:]
        avg_us[k] = sum(e - b for b, e in last) / len(last) / 1e3

    fetch, write = per_kernel("FETCH_SIZE"), per_kernel("WRITE_SIZE")
    fs, ws = CALIBRATION_KIB / fetch[COPY_KERNEL], CALIBRATION_KIB / write[COPY_KERNEL]
    out = {}
    for k in fetch:
        if not (k.startswith("_ZN4attn") or k.startswith("attn::")) or "clock_probe" in k:
            continue
        out[kernel_label(k)] = {
            "kernel": kernel_label(k), "avg_us": avg_us.get(k),
            "hbm_bytes_per_launch": (fetch[k] * fs + write[k] * ws) * 1024,
            "fetch_kib_raw": fetch[k], "write_kib_raw": write[k],
            "fetch_scale": fs, "write_scale": ws}
    return out


def traffic_from(indir: str, path: str = TRAFFIC_FILE):
    """Write the traffic file from the counter runs under `indir` (the runs of
    TRAFFIC_RUNS that are there), stamped with the current kernel-source hash."""
    def has(run):
        return all(os.path.exists(os.path.join(indir, f"{run}_{p}", f))
                   for p, f in (("FETCH_SIZE", "run_counter_collection.csv"),
                                ("WRITE_SIZE", "run_counter_collection.csv"),
                                ("trace", "run_kernel_trace.csv")))

    def pick(ks, prefix, suffix=""):
        hits = [v for k, v in ks.items()
                if (k == prefix or k.startswith(prefix + "<")) and k.endswith(suffix)]
        if len(hits) != 1:
            raise SystemExit(f"traffic: {len(hits)} kernels match {prefix}...{suffix}")
        return hits[0]

    def call(*parts):
        return {"kernel": " + ".join(p["kernel"] for p in parts),
                "avg_us": sum(p["avg_us"] for p in parts),
                "hbm_bytes_per_launch": sum(p["hbm_bytes_per_launch"] for p in parts)}

    rec = {"source_hash": kernel_source_hash(),
           "note": "HBM bytes per launch (per call where one call launches several kernels), "
                   "from rocprofv3 FETCH_SIZE and WRITE_SIZE scaled by a 512 MiB copy",
           "kernels": {}}
    kern = rec["kernels"]
    if has("step"):
        s = counter_run(indir, "step")
        kern["fwd"] = pick(s, "fwd_mfma_kernel")
        kern["bwd_dq"] = pick(s, "bwd_dq_kernel")
        kern["bwd_dkdv"] = pick(s, "bwd_dkdv_kernel")
    for n in (2, 3, 4):
        if has(f"fwd{n}"):
            f = counter_run(indir, f"fwd{n}")
            kern[f"fwd_workload{n}"] = next(v for k, v in f.items() if k.startswith("fwd_mfma"))
    if has("bwd4"):
        b = counter_run(indir, "bwd4")
        dq, kv = pick(b, "bwd_dq_kernel"), pick(b, "bwd_dkdv_kernel")
        kern["bwd_workload4"] = call(dq, kv)
        rec["bwd_workload4_kernels"] = {"bwd_dq": dq, "bwd_dkdv": kv}
    if has("decode"):
        c = counter_run(indir, "decode")
        sp, cb = pick(c, "fwd_split_kernel"), pick(c, "split_combine_kernel")
        kern["splitkv_decode"] = call(sp, cb)
        rec["splitkv_decode_kernels"] = {"fwd_split": sp, "split_combine": cb}
    if has("sparse"):
        c = counter_run(indir, "sparse")
        cp = pick(c, "sparse_compact_kernel")
        fw = next(v for k, v in c.items() if k.startswith("fwd_mfma") and k.endswith(", 1>"))
        kern["blocksparse_local_global"] = call(cp, fw)
        rec["blocksparse_kernels"] = {"sparse_compact": cp, "fwd": fw}
    if has("varlen"):
        c = counter_run(indir, "varlen")
        kern["varlen_docs"] = next(v for k, v in c.items()
                                   if k.startswith("fwd_mfma") and k.endswith(", 2>"))
        rec["varlen_backward_kernels"] = {k: v for k, v in c.items() if k.startswith("bwd")}
    if not kern:
        raise SystemExit(f"traffic: no complete counter run under {indir}")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    for k, v in kern.items():
        print(f"{k:26s} {v['avg_us']:9.1f} us {v['hbm_bytes_per_launch'] / 1e9:7.3f} GB  {v['kernel']}")


def roofline_mfma(tflops: float, traffic_key: str | None):
    """A sweep entry's roofline: algorithmic TFLOP/s against the dense bf16
    peak, with the HBM bytes per call from the counters when they were taken
    on the current sources."""
    return {"bound": "mfma", "achieved": round(tflops, 1), "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(traffic_key) if traffic_key else None}


class ClockProbe:
    """The shader clock of each XCD while the steps run.  attn_probe_clock's
    one-wave workgroups (8: one per XCD) spin on a second stream for a fixed
    real-time window beside the steps, each comparing its XCD's shader-clock
    counter with the 100 MHz real-time counter.  Under sustained matrix-core
    load the board lowers its clock to hold its power limit and raises it
    again within microseconds once the load stops, so the probe has to overlap
    the steps: probes launched between kernels read the idle 2.4 GHz.  (The
    SMI library's graphics-clock fields read 200-700 MHz during such steps on
    these boards, and loading it slowed the steps by 4-5%, so it is not
    used.)"""

    NWG = 8

    def __init__(self, dev, window_ms: float):
        import torch

        self.buf = torch.zeros(2 * self.NWG, dtype=torch.int64, device=dev)
        self.stream = torch.cuda.Stream(dev)  # default priority
        self.window_ms = min(max(window_ms, 0.01), 2000.0)

    def start(self):
        import exact_attention_87_amd as ea

        st = ea.attn_probe_clock(self.buf.data_ptr(), self.NWG, int(self.window_ms * 1e5),
                                 self.stream.cuda_stream)
        if st != ea.ATTN_OK:
            raise ea.AttnError(st, "attn_probe_clock")

    def summary(self):
        """After the device has been synchronised."""
        v = self.buf.cpu().tolist()
        mhz = [v[2 * i] / v[2 * i + 1] * 100.0 for i in range(self.NWG) if v[2 * i + 1] > 0]
        if not mhz:
            return {"source": "attn_probe_clock", "samples": 0}
        return {"mean_mhz": round(sum(mhz) / len(mhz), 1), "min_mhz": round(min(mhz), 1),
                "max_mhz": round(max(mhz), 1), "per_xcd_mhz": [round(x, 1) for x in mhz],
                "probe_ms": round(v[1] / 1e5, 2),
                "source": "attn_probe_clock: shader-clock counter against the 100 MHz real-time "
                          "counter, one wave per XCD on a second stream beside the steps"}


HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5  # hipDeviceAttributeClockRate (kHz), hip_runtime_api.h


def hip_version_string():
    """HIP version of the installed toolchain, from its version header."""
    import re

    try:
        with open("/opt/rocm/include/hip/hip_version.h") as f:
            text = f.read()
    except OSError:
        return None
    v = dict(re.findall(r"#define HIP_VERSION_(MAJOR|MINOR|PATCH|GITHASH)\s+\"?([^\s\"]*)", text))
    if not all(k in v for k in ("MAJOR", "MINOR", "PATCH")):
        return None
    return f"HIP version: {v['MAJOR']}.{v['MINOR']}.{v['PATCH']}" + (
        f"-{v['GITHASH']}" if v.get("GITHASH") else "")


def max_sclk_mhz(index: int):
    """Peak engine clock of device `index` from the HIP runtime torch has
    loaded (by soname, so no second runtime is opened).  Asked in-process:
    a child tool (rocminfo) would, under a profiler that preloads its library
    into every process, initialise the GPU in the child before it execs."""
    import ctypes

    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        val = ctypes.c_int(0)
        rc = hip.hipDeviceGetAttribute(ctypes.byref(val), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE, index)
    except (OSError, AttributeError):
        return None
    return val.value // 1000 if rc == 0 and val.value > 0 else None


def environment(dev):
    """Where the numbers were taken: device, software versions, host.  Read
    from files and in-process calls only: this process holds the GPU, and no
    child program is started."""
    import torch

    props = torch.cuda.get_device_properties(dev)
    env = {"gpu": torch.cuda.get_device_name(dev), "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count,
           "device_memory_bytes": props.total_memory, "torch": torch.__version__,
           "torch_hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    env["hipcc"] = hip_version_string()
    try:
        with open("/proc/cpuinfo") as f:
            env["host_cpu"] = next((l.split(":", 1)[1].strip() for l in f if
                                    l.startswith("model name")), None)
    except OSError:
        env["host_cpu"] = None
    env["host_cpus"] = os.cpu_count()
    # the peak recomputed from this device: CUs x 4096 bf16 FLOP/clk/CU x its
    # peak engine clock
    mhz = max_sclk_mhz(dev.index if dev.index is not None else 0)
    env["max_sclk_mhz"] = mhz
    env["peak_bf16_tflops_at_max_sclk"] = (
        round(props.multi_processor_count * 4096 * mhz * 1e6 / 1e12, 1) if mhz else None)
    return env


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle (forward + backward) on whole (batch, head) slices of
    the workload, one after another until the time budget is spent."""
    import oracle

    import attn_inputs

    q, k, v, do = attn_inputs.make_workload(w, with_dout=True)
    slices = w.B * w.Hkv
    per_slice = (fwd_flops(1, w.Hq // w.Hkv, w.N, w.d, w.causal) * 3.5)  # fwd + bwd (4 + 10)
    done = 0
    t0 = time.perf_counter()
    while done < slices and (time.perf_counter() - t0) < budget_s:
        oracle.bwd_slices(q, k, v, do, [done], causal=w.causal)
        done += 1
    dt = time.perf_counter() - t0
    return {
        "value": per_slice * done / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.omp_threads(),
        "kind": "oracle",
        "sample": f"{done} of {slices} (batch, head) slices of the same workload, "
                  f"full fp64 forward+backward each, {dt:.1f} s",
        "seconds": round(dt, 3),
        "host_cpus": os.cpu_count(),
    }


def forward_only(w, args, dev):
    """Forward of one workload: K timed launches of attn_fwd (events on the stream)."""
    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    q, k, v = (t.to(dev) for t in attn_inputs.make_workload(w, with_dout=False))
    o, lse = ea.fwd(q, k, v, causal=w.causal)
    warm_up(lambda: ea.fwd(q, k, v, causal=w.causal, out=o, lse=lse), args.warmup)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        ea.fwd(q, k, v, causal=w.causal, out=o, lse=lse)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    fl = fwd_flops(w.B, w.Hq, w.N, w.d, w.causal)
    print(json.dumps({
        "metric": "attention forward TFLOP/s on 1 MI355X", "value": round(fl / ms / 1e9, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "kernel_ms": round(ms, 5),
        "frac_of_peak": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "higher_is_better": True,
        "dtype": w.dtype, "data": "synthetic",
        "roofline": {"bound": "mfma", "achieved": round(fl / ms / 1e9, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(fl / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(f"fwd_workload{args.fwd_only}"), "kernel": "fwd"},
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "q_mult": w.q_mult, "seed": w.seed}}), flush=True)


def backward_only(w, args, dev):
    """attn_bwd alone on workload w (the forward's O and LSE precomputed): K timed
    calls, HIP events on the stream.  Algorithmic FLOPs 10*B*Hq*N^2*d, halved
    for causal (the dQ stage's recomputed S and dP are executed, not counted)."""
    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    q, k, v, do = (t.to(dev) for t in attn_inputs.make_workload(w, with_dout=True))
    o, lse = ea.fwd(q, k, v, causal=w.causal)
    ws = torch.empty(max(ea.attn_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, ea.ATTN_BF16),
                         256), device=dev, dtype=torch.uint8)
    grads = [torch.empty_like(t) for t in (q, k, v)]
    sp = torch.cuda.current_stream(dev).cuda_stream

    def call():
        st = ea.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         do.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                         grads[2].data_ptr(), ws.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
                         int(w.causal), w.d ** -0.5, ea.ATTN_BF16, sp)
        if st != ea.ATTN_OK:
            raise ea.AttnError(st, "attn_bwd")

    warm_up(call, args.warmup)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    fl = 2.5 * fwd_flops(w.B, w.Hq, w.N, w.d, w.causal)
    tf = fl / ms / 1e9
    print(json.dumps({
        "metric": "attention backward TFLOP/s on 1 MI355X", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "kernel_ms": round(ms, 5),
        "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "higher_is_better": True,
        "dtype": w.dtype, "data": "synthetic",
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(f"bwd_workload{args.bwd_only}"),
                     "kernel": "attn_bwd (dQ stage with statistics + dK/dV stage)"},
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "q_mult": w.q_mult, "seed": w.seed}}), flush=True)


def calibration_copy(mib, dev):
    """One plain device copy of `mib` MiB: a transfer of known size that
    scales the HBM byte counters of a profiling run."""
    import torch

    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def splitkv_visible_pairs(Nq, Nk, causal):
    """(query, key) pairs the bottom-right aligned mask leaves visible per head."""
    if not causal:
        return Nq * Nk
    return sum(max(0, min(Nk, i + 1 + Nk - Nq)) for i in range(Nq))


def splitkv_case(cw, dev, steps, warmup, num_splits=0):
    """attn_fwd_splitkv on one cache workload: `steps` timed calls (split kernel
    + merge kernel), HIP events on the launch stream.  HBM-bound: the
    algorithmic bytes are K and V once, plus Q, O and LSE."""
    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    q, k, v = (t.to(dev) for t in attn_inputs.make_cache_workload(cw))
    o = torch.empty_like(q)
    lse = torch.empty((cw.B, cw.Hq, cw.Nq), device=dev, dtype=torch.float32)
    nbytes = ea.attn_fwd_splitkv_workspace_bytes(cw.B, cw.Hq, cw.Hkv, cw.Nq, cw.Nk, cw.d,
                                                 num_splits)
    ws = torch.empty(max(nbytes, 256), device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    scale = 1.0 / math.sqrt(cw.d)

    def call():
        st = ea.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), ws.data_ptr(), cw.B, cw.Hq, cw.Hkv, cw.Nq, cw.Nk,
                                 cw.d, int(cw.causal), scale, num_splits, ea.ATTN_BF16,
                                 stream.cuda_stream)
        if st != ea.ATTN_OK:
            raise ea.AttnError(st, "attn_fwd_splitkv")

    warm_up(call, warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    byts = (2 * cw.B * cw.Hkv * cw.Nk * cw.d * 2 + 2 * cw.B * cw.Hq * cw.Nq * cw.d * 2
            + cw.B * cw.Hq * cw.Nq * 4)
    flops = 4.0 * cw.B * cw.Hq * cw.d * splitkv_visible_pairs(cw.Nq, cw.Nk, cw.causal)
    gbs = byts / (ms / 1e3) / 1e9
    return {"us": round(ms * 1e3, 2), "gbs": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "tflops": round(flops / (ms / 1e3) / 1e12, 1), "algorithmic_bytes": byts,
            "num_splits": ea.attn_fwd_splitkv_num_splits(cw.B, cw.Hq, cw.Hkv, cw.Nq, cw.Nk, cw.d,
                                                         num_splits)}


def sparse_visible_pairs(mask, N, bq, bk, causal):
    """(query, key) pairs a block mask (and the causal rule) leaves visible,
    summed over the mask's heads."""
    import numpy as np

    nbq, nbk = mask.shape[1], mask.shape[2]
    qb = np.arange(nbq)[:, None]
    t = np.arange(nbk)[None, :]
    q0, q1 = qb * bq, np.minimum((qb + 1) * bq, N)
    k0, k1 = t * bk, np.minimum((t + 1) * bk, N)
    if not causal:
        pairs = (q1 - q0) * (k1 - k0)
    else:
        # rows i in [q0, q1) see keys [k0, min(k1, i + 1)): sum over the rows
        pairs = np.zeros((nbq, nbk), np.int64)
        for i in range(bq):
            row = q0 + i
            pairs += np.where(row < q1, np.clip(np.minimum(k1, row + 1) - k0, 0, None), 0)
    return int((mask.astype(np.int64) * pairs[None]).sum())


def sparse_case(sw, dev, steps, warmup):
    """attn_fwd_blocksparse on a block-sparse workload (mask compaction +
    forward, one call), timed with HIP events on the launch stream, and the
    dense forward of the same shape for comparison.  TFLOP/s count the
    visible (query, key) pairs only: 4*d per pair."""
    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    q, k, v = (t.to(dev) for t in attn_inputs.make(sw.B, sw.Hq, sw.Hkv, sw.N, sw.d, "bf16",
                                                    seed=sw.seed))
    mask_np = attn_inputs.sparse_mask(sw)
    mask = torch.from_numpy(mask_np).to(dev)
    o, lse = ea.fwd_blocksparse(q, k, v, mask, causal=sw.causal)
    ws = torch.empty(ea.attn_fwd_blocksparse_workspace_bytes(sw.Hq, sw.N, mask.shape[0]),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        warm_up(fn, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: ea.fwd_blocksparse(q, k, v, mask, causal=sw.causal, out=o, lse=lse,
                                          workspace=ws))
    ms_dense = timed(lambda: ea.fwd(q, k, v, causal=sw.causal, out=o, lse=lse))
    pairs = sw.B * sparse_visible_pairs(mask_np, sw.N, ea.SPARSE_BLOCK_Q, ea.SPARSE_BLOCK_K,
                                        sw.causal)
    dense_pairs = sw.B * sw.Hq * (sw.N * (sw.N + 1) // 2 if sw.causal else sw.N * sw.N)
    tf = 4.0 * sw.d * pairs / (ms / 1e3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "visible_fraction": round(pairs / dense_pairs, 4), "dense_ms": round(ms_dense, 4),
            "speedup_vs_dense": round(ms_dense / ms, 2)}


def varlen_case(vw, dev, steps, warmup):
    """attn_fwd_varlen on a packed document batch, timed with HIP events, and
    the same documents padded to the longest one through attn_fwd for
    comparison.  TFLOP/s count the visible pairs of each document only."""
    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    lengths = attn_inputs.varlen_lengths(vw)
    q, k, v, cu = (t.to(dev) for t in attn_inputs.make_varlen(vw.Hq, vw.Hkv, lengths, vw.d,
                                                               seed=vw.seed))
    mx = max(lengths)
    o, lse = ea.fwd_varlen(q, k, v, cu, mx, causal=vw.causal)
    nseq = len(lengths)
    qp = torch.zeros((nseq, vw.Hq, mx, vw.d), device=dev, dtype=q.dtype)
    kp = torch.zeros((nseq, vw.Hkv, mx, vw.d), device=dev, dtype=q.dtype)
    vp_ = torch.zeros_like(kp)
    for s_, (a, n) in enumerate(zip(cu.tolist()[:-1], lengths)):
        qp[s_, :, :n] = q[:, a:a + n]
        kp[s_, :, :n] = k[:, a:a + n]
        vp_[s_, :, :n] = v[:, a:a + n]
    op, lp = ea.fwd(qp, kp, vp_, causal=vw.causal)
    stream = torch.cuda.current_stream(dev)

    def timed(fn):
        warm_up(fn, warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: ea.fwd_varlen(q, k, v, cu, mx, causal=vw.causal, out=o, lse=lse))
    ms_pad = timed(lambda: ea.fwd(qp, kp, vp_, causal=vw.causal, out=op, lse=lp))
    # backward of the same packed batch (statistics, dK/dV and dQ launches)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(vw.seed + 1)).to(
        dev, dtype=q.dtype)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(ea.attn_bwd_workspace_bytes(1, vw.Hq, vw.Hkv, vw.T, vw.d, ea.ATTN_BF16),
                         256), device=dev, dtype=torch.uint8)
    ms_bwd = timed(lambda: ea.bwd_varlen(q, k, v, o, lse, do, cu, mx, causal=vw.causal,
                                         workspace=ws, dq=dq, dk=dk, dv=dv))
    pairs = sum(n * (n + 1) // 2 if vw.causal else n * n for n in lengths) * vw.Hq
    tf = 4.0 * vw.d * pairs / (ms / 1e3) / 1e12
    tfb = 10.0 * vw.d * pairs / (ms_bwd / 1e3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "sequences": nseq, "longest": mx, "padded_ms": round(ms_pad, 4),
            "speedup_vs_padded": round(ms_pad / ms, 2), "bwd_ms": round(ms_bwd, 4),
            "bwd_tflops": round(tfb, 1), "bwd_frac_of_peak": round(tfb / PEAK_BF16_TFLOPS, 4)}


def varlen_only(name, args, dev):
    import attn_inputs

    vw = attn_inputs.VARLEN_WORKLOADS[name]
    r = varlen_case(vw, dev, args.steps, args.warmup)
    print(json.dumps({
        "metric": "packed variable-length attention forward TFLOP/s on 1 MI355X",
        "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "roofline": {"bound": "mfma", "achieved": r["tflops"], "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": r["frac_of_peak"],
                     "traffic": load_traffic("varlen_" + name),
                     "kernel": "fwd_mfma_pipe (one launch; 4*d FLOP per visible pair)"},
        "detail": r,
        "config": {"workload": vw.name, "Hq": vw.Hq, "Hkv": vw.Hkv, "T": vw.T, "d": vw.d,
                   "causal": vw.causal, "seed": vw.seed}}), flush=True)


def sparse_only(name, args, dev):
    import attn_inputs

    sw = attn_inputs.SPARSE_WORKLOADS[name]
    r = sparse_case(sw, dev, args.steps, args.warmup)
    print(json.dumps({
        "metric": "block-sparse attention forward TFLOP/s (visible pairs) on 1 MI355X",
        "value": r["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms"], "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "roofline": {"bound": "mfma", "achieved": r["tflops"], "peak": round(PEAK_BF16_TFLOPS, 1),
                     "unit": "TFLOP/s", "frac": r["frac_of_peak"],
                     "traffic": load_traffic("blocksparse_" + name),
                     "kernel": "sparse_compact + fwd_mfma_pipe (one call; 4*d FLOP per visible pair)"},
        "detail": r,
        "config": {"workload": sw.name, "B": sw.B, "Hq": sw.Hq, "Hkv": sw.Hkv, "N": sw.N,
                   "d": sw.d, "causal": sw.causal, "seed": sw.seed}}), flush=True)


def splitkv_only(name, args, dev):
    import attn_inputs

    cw = attn_inputs.CACHE_WORKLOADS[name]
    r = splitkv_case(cw, dev, args.steps, args.warmup)
    print(json.dumps({
        "metric": "split-K/V attention forward GB/s on 1 MI355X (HBM-bound)",
        "value": r["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(r["us"] / 1e3, 5), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "roofline": {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": r["frac_of_hbm"], "traffic": load_traffic("splitkv_" + name),
                     "kernel": "fwd_split + split_combine (one call)"},
        "detail": r,
        "config": {"workload": cw.name, "B": cw.B, "Hq": cw.Hq, "Hkv": cw.Hkv, "Nq": cw.Nq,
                   "Nk": cw.Nk, "d": cw.d, "causal": cw.causal, "seed": cw.seed}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before the timed ones (the GPU's clocks ramp up from idle "
                         "over tens of milliseconds)")
    ap.add_argument("--prewarm-ms", type=float, default=60.0,
                    help="before the warm-up steps, run untimed steps until the GPU has been busy "
                         "this long (reported as prewarm_ms; 0 disables)")
    ap.add_argument("--clock", choices=("after", "timed", "off"), default="after",
                    help="measure the shader clock (attn_probe_clock on a second stream) beside "
                         "the same steps right after the timed region (default), beside the timed "
                         "steps themselves, or not at all")
    ap.add_argument("--clock-ms", type=float, default=300.0,
                    help="length of the clock window after the timed region")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="time budget of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the forward sweep")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--fwd-only", type=int, default=0, metavar="ID",
                    help="time only the forward of workload ID (1-5) and print its JSON line")
    ap.add_argument("--bwd-only", type=int, default=0, metavar="ID",
                    help="time only attn_bwd on workload ID (1-5; fp32 workload 1 has none)")
    ap.add_argument("--sparse-only", default="", metavar="NAME",
                    help="time only the block-sparse forward of workload NAME (local_global)")
    ap.add_argument("--varlen-only", default="", metavar="NAME",
                    help="time only the packed variable-length forward of workload NAME (docs)")
    ap.add_argument("--splitkv-only", default="", metavar="NAME",
                    help="time only the split-K/V forward of cache workload NAME "
                         "(decode, append) and print its JSON line")
    ap.add_argument("--traffic-from", default="", metavar="DIR",
                    help="no GPU run: write profiles/traffic.json from the rocprofv3 counter "
                         "runs under DIR (named as in TRAFFIC_RUNS)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; use --gpus 1"}))
        print("bench.py: only --gpus 1 is supported (single-GPU kernel library)", file=sys.stderr)
        sys.exit(2)

    import torch

    import attn_inputs
    import exact_attention_87_amd as ea

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    ea.lib()  # fail loudly if the HIP library is missing

    if args.fwd_only or args.bwd_only or args.splitkv_only or args.sparse_only or args.varlen_only:
        calibration_copy(args.copy_mib, dev)
    if args.fwd_only:
        forward_only(attn_inputs.WORKLOADS[args.fwd_only], args, dev)
        return
    if args.bwd_only:
        if args.bwd_only == 1:
            print("bench.py: workload 1 is the fp32 forward parity case; it has no backward",
                  file=sys.stderr)
            sys.exit(2)
        backward_only(attn_inputs.WORKLOADS[args.bwd_only], args, dev)
        return
    if args.splitkv_only:
        splitkv_only(args.splitkv_only, args, dev)
        return
    if args.sparse_only:
        sparse_only(args.sparse_only, args, dev)
        return
    if args.varlen_only:
        varlen_only(args.varlen_only, args, dev)
        return

    env = environment(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    w = attn_inputs.WORKLOADS[5]
    B, Hq, Hkv, N, d = w.B, w.Hq, w.Hkv, w.N, w.d
    scale = 1.0 / math.sqrt(d)
    causal = int(w.causal)
    q, k, v, do = (t.to(dev) for t in attn_inputs.make_workload(w, with_dout=True))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), device=dev, dtype=torch.float32)
    stats = torch.empty(ea.attn_bwd_workspace_bytes(B, Hq, Hkv, N, d, ea.ATTN_BF16) // 4,
                        device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    BF = ea.ATTN_BF16

    def check(st, what):
        if st != ea.ATTN_OK:
            raise ea.AttnError(st, what)

    launches = [
        ("fwd", lambda: check(ea.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), B, Hq, Hkv, N, d, causal, scale, BF,
                                          sp), "attn_fwd")),
        ("bwd_dq", lambda: check(ea.attn_bwd_dq_stats(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
            stats.data_ptr(), dq.data_ptr(), B, Hq, Hkv, N, d, causal, scale, BF, sp),
            "attn_bwd_dq_stats")),
        ("bwd_dkdv", lambda: check(ea.attn_bwd_dkdv(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), stats.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, causal, scale, BF, sp),
            "attn_bwd_dkdv")),
    ]
    f1 = fwd_flops(B, Hq, N, d, w.causal)  # = 4*B*H*N^2*d/2
    unit = f1 / 4.0  # B*H*N^2*d/2
    algo = {  # algorithmic FLOPs and HBM bytes per launch
        "fwd": {"flops": 4 * unit, "bytes": (2 * B * Hq + 2 * B * Hkv) * N * d * 2 + B * Hq * N * 4},
        # dQ stage: Q, dO, O read, dQ written, K, V read; LSE read, statistics written
        "bwd_dq": {"flops": 2 * unit,
                   "bytes": (4 * B * Hq + 2 * B * Hkv) * N * d * 2 + 3 * B * Hq * N * 4},
        "bwd_dkdv": {"flops": 8 * unit,
                     "bytes": (2 * B * Hq + 4 * B * Hkv) * N * d * 2 + 2 * B * Hq * N * 4},
    }
    step_flops = 14 * unit

    def step(events=None):
        for i, (_, fn) in enumerate(launches):
            fn()
            if events is not None:
                events[i].record(stream)

    # Pre-warm, reported separately: untimed steps until the GPU has been busy
    # for --prewarm-ms, so the clocks have left idle whatever W is; then
    # exactly W untimed warm-up steps, then the K timed ones.
    t_pw = time.perf_counter()
    prewarm_steps = 0
    while (time.perf_counter() - t_pw) * 1e3 < args.prewarm_ms:
        for _ in range(8):
            step()
        prewarm_steps += 8
        torch.cuda.synchronize()
    prewarm_ms = (time.perf_counter() - t_pw) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    calibration_copy(args.copy_mib, dev)

    K = args.steps
    # HIP events recorded between the launches of every fifth timed step give
    # each kernel's duration; the steps in between run without them.  Each
    # event adds a dispatch gap of about 6 us before the next kernel (measured
    # in a kernel trace), so probing fewer steps keeps the instrumentation's
    # share of the timed region small.
    probed = list(range(0, K, 5))
    evs = {s: [torch.cuda.Event(enable_timing=True) for _ in launches] for s in probed}
    start = {s: torch.cuda.Event(enable_timing=True) for s in probed}
    # The clock probe runs beside the same steps for --clock-ms right after the
    # timed region (the default: steps beside it ran at the timed rate), or
    # beside the timed steps themselves (--clock timed: its launch on a second
    # queue made a 30-step timed region 13% slower).
    clock = None
    if args.clock == "timed":
        est_ms = prewarm_ms / max(prewarm_steps, 1) * K  # this box's pre-warm rate
        clock = ClockProbe(dev, 0.9 * est_ms)
    torch.cuda.synchronize()
    if clock is not None:
        clock.start()
    t0 = time.perf_counter()
    for s in range(K):
        if s in start:
            start[s].record(stream)
            step(evs[s])
        else:
            step()
    stream.synchronize()
    wall = time.perf_counter() - t0
    torch.cuda.synchronize()
    ms_per_step = wall * 1e3 / K
    # device memory the step holds (the library allocates none itself: inputs,
    # outputs, statistics workspace)
    peak_mem = torch.cuda.max_memory_allocated(dev)
    beside_ms = None
    if args.clock == "after":
        clock = ClockProbe(dev, args.clock_ms)
        clock.start()
        t1 = time.perf_counter()
        n1 = 0
        while (time.perf_counter() - t1) * 1e3 < args.clock_ms:
            for _ in range(32):
                step()
            n1 += 32
            stream.synchronize()  # the steps' stream only: the probe is still running
        beside_ms = (time.perf_counter() - t1) * 1e3 / n1
        torch.cuda.synchronize()  # now the probe too

    kern_ms = {name: 0.0 for name, _ in launches}
    for s in probed:
        prev = start[s]
        for i, (name, _) in enumerate(launches):
            kern_ms[name] += prev.elapsed_time(evs[s][i]) / len(probed)
            prev = evs[s][i]
    gpu_ms = sum(kern_ms.values())

    kernels = {}
    for name, _ in launches:
        t = kern_ms[name] / 1e3
        rec = {"ms": round(kern_ms[name], 5)}
        if algo[name]["flops"] > 0:
            rec["tflops"] = round(algo[name]["flops"] / t / 1e12, 2)
            rec["frac_of_peak"] = round(algo[name]["flops"] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        rec["gbs"] = round(algo[name]["bytes"] / t / 1e9, 1)
        kernels[name] = rec
    dom = max(kern_ms, key=kern_ms.get)
    t_dom = kern_ms[dom] / 1e3
    if algo[dom]["flops"] > 0:
        ach = algo[dom]["flops"] / t_dom / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": round(PEAK_BF16_TFLOPS, 1),
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = algo[dom]["bytes"] / t_dom / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = load_traffic(dom)
    roof["kernel"] = dom

    # forward sweep over the other workloads (parity-tested separately)
    sweep = {}
    if not args.no_sweep:
        cases = [attn_inputs.WORKLOADS[i] for i in (2, 3, 4)] + [
            attn_inputs.Workload("noncausal_bf16_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, False,
                                 "bf16", seed=6),
            attn_inputs.Workload("noncausal_bf16_B1_H32_N8192_d128", 1, 32, 32, 8192, 128, False,
                                 "bf16", seed=7),
            attn_inputs.Workload("causal_fp16_B1_H32_N8192_d128", 1, 32, 32, 8192, 128, True,
                                 "fp16", seed=8),
            attn_inputs.Workload("noncausal_bf16_B1_H16_N8192_d256", 1, 16, 16, 8192, 256, False,
                                 "bf16", seed=9),
        ]
        for cw in cases:
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            cq, ck, cv = (t.to(dev) for t in attn_inputs.make_workload(cw, with_dout=False))
            co, cl = ea.fwd(cq, ck, cv, causal=cw.causal)
            warm_up(lambda: ea.fwd(cq, ck, cv, causal=cw.causal, out=co, lse=cl), 5)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 25
            e0.record(stream)
            for _ in range(reps):
                ea.fwd(cq, ck, cv, causal=cw.causal, out=co, lse=cl)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = fwd_flops(cw.B, cw.Hq, cw.N, cw.d, cw.causal) / (ms / 1e3) / 1e12
            wid = next((i for i, x in attn_inputs.WORKLOADS.items() if x.name == cw.name), None)
            sweep[cw.name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                              "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "roofline": roofline_mfma(tf, f"fwd_workload{wid}" if wid else None),
                              "peak_mem_bytes": torch.cuda.max_memory_allocated(dev)}
            del cq, ck, cv, co, cl
        torch.cuda.synchronize()

    # backward sweep (attn_bwd alone, back-to-back calls; parity-tested separately)
    bwd_sweep = {}
    if not args.no_sweep:
        bcases = [
            attn_inputs.Workload("causal_gqa_bf16_B1_Hq32_Hkv8_N16384_d128", 1, 32, 8, 16384, 128,
                                 True, "bf16", seed=4),
            attn_inputs.Workload("noncausal_bf16_B2_H32_N4096_d128", 2, 32, 32, 4096, 128, False,
                                 "bf16", seed=6),
            attn_inputs.Workload("causal_bf16_B4_H32_N4000_d128", 4, 32, 32, 4000, 128, True,
                                 "bf16", seed=3),
            attn_inputs.Workload("noncausal_bf16_B1_H16_N8192_d256", 1, 16, 16, 8192, 256, False,
                                 "bf16", seed=9),
            # grouped-query heads at a short length: 128 key blocks x kv heads, so the
            # dK/dV stage splits each group's query heads over 4 workgroups
            attn_inputs.Workload("causal_gqa_bf16_B1_Hq32_Hkv8_N2048_d128", 1, 32, 8, 2048, 128,
                                 True, "bf16", seed=12),
        ]
        for cw in bcases:
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            cq, ck, cv, cdo = (t.to(dev) for t in attn_inputs.make_workload(cw, with_dout=True))
            co, cl = ea.fwd(cq, ck, cv, causal=cw.causal)
            cws = torch.empty(ea.attn_bwd_workspace_bytes(cw.B, cw.Hq, cw.Hkv, cw.N, cw.d,
                                                          ea.ATTN_BF16), device=dev,
                              dtype=torch.uint8)
            grads = [torch.empty_like(t) for t in (cq, ck, cv)]

            def bwd_call():
                check(ea.attn_bwd(cq.data_ptr(), ck.data_ptr(), cv.data_ptr(), co.data_ptr(),
                                  cl.data_ptr(), cdo.data_ptr(), grads[0].data_ptr(),
                                  grads[1].data_ptr(), grads[2].data_ptr(), cws.data_ptr(), cw.B,
                                  cw.Hq, cw.Hkv, cw.N, cw.d, int(cw.causal), cw.d ** -0.5,
                                  ea.ATTN_BF16, sp), "attn_bwd")

            warm_up(bwd_call, 3)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record(stream)
            for _ in range(reps):
                bwd_call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            tf = 2.5 * fwd_flops(cw.B, cw.Hq, cw.N, cw.d, cw.causal) / (ms / 1e3) / 1e12
            key = "bwd_workload4" if cw.name == "causal_gqa_bf16_B1_Hq32_Hkv8_N16384_d128" else None
            bwd_sweep[cw.name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                  "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "roofline": roofline_mfma(tf, key),
                                  "peak_mem_bytes": torch.cuda.max_memory_allocated(dev)}
            del cq, ck, cv, cdo, co, cl, cws, grads
        torch.cuda.synchronize()

    # split-K/V forward on the key/value-cache workloads (parity-tested separately)
    splitkv = {}
    if not args.no_sweep:
        for name, cw in attn_inputs.CACHE_WORKLOADS.items():
            r = splitkv_case(cw, dev, steps=20, warmup=3)
            r["roofline"] = {"bound": "hbm", "achieved": r["gbs"], "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": r["frac_of_hbm"],
                             "traffic": load_traffic("splitkv_" + name)}
            splitkv[cw.name] = r
        torch.cuda.synchronize()

    # block-sparse forward (parity-tested separately)
    blocksparse = {}
    if not args.no_sweep:
        for name, sw in attn_inputs.SPARSE_WORKLOADS.items():
            r = sparse_case(sw, dev, steps=10, warmup=3)
            r["roofline"] = roofline_mfma(r["tflops"], "blocksparse_" + name)
            blocksparse[sw.name] = r
        torch.cuda.synchronize()

    # packed variable-length forward (parity-tested separately)
    varlen = {}
    if not args.no_sweep:
        for name, vw in attn_inputs.VARLEN_WORKLOADS.items():
            r = varlen_case(vw, dev, steps=10, warmup=3)
            r["roofline"] = roofline_mfma(r["tflops"], "varlen_" + name)
            varlen[vw.name] = r
        torch.cuda.synchronize()

    cpu = cpu_baseline(w, args.cpu_seconds) if args.cpu_seconds > 0 else None
    value = step_flops / (ms_per_step / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup, "prewarm_ms": round(prewarm_ms, 1), "prewarm_steps": prewarm_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d,
                   "causal": bool(causal), "scale": scale, "seed": w.seed,
                   "step": "attn_fwd + attn_bwd_dq_stats + attn_bwd_dkdv"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "peak_tflops_bf16": round(PEAK_BF16_TFLOPS, 1),
        "gpu_ms_per_step": round(gpu_ms, 5),
        "roofline": roof,
        "kernels": kernels,
        "forward_sweep": sweep,
        "backward_sweep": bwd_sweep,
        "splitkv": splitkv,
        "blocksparse": blocksparse,
        "varlen": varlen,
        "cpu_baseline": cpu,
        "peak_mem_bytes": peak_mem,
        "sclk": dict(clock.summary(), window=(
            "beside the timed steps" if args.clock == "timed" else
            f"{args.clock_ms:.0f} ms beside the same steps right after the timed region"),
            ms_per_step_beside_probe=None if beside_ms is None else round(beside_ms, 5))
        if clock is not None else None,
        "env": env,
        "device": env["gpu"],
        "torch": torch.__version__,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
