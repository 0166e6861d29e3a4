#!/usr/bin/env python3
"""Benchmark of the selective-scan forward pass on one MI355X.

One step = one call of ssm_selective_scan_fwd over the whole Mamba-1.3B-shaped
layer workload (batch 4, L 4096, dim 4096, dstate 16, bf16 I/O, fp32 state):
every stage of the path (loads, softplus, discretisation, scan, read-out, skip,
gate, bf16 store) runs inside the timed region, with inputs already in HBM.

Defaults: 50 untimed warm-up calls (the GPU clock ramps up over the first few
milliseconds), then 200 timed calls.  Prints one JSON line.  ``value`` is state updates per second (B*L*D*N / step time);
``roofline`` reports the dominant kernel against its binding roof, ``hbm`` the
achieved algorithmic GB/s against the 8 TB/s HBM peak, and ``cpu_baseline`` the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan state updates/sec (B·L·D·N) + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
# fp32 VALU lane-operation rate without packed-fp32 instructions:
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# minimal VALU operations per state update of the diagonal-A method:
# dt*A (mul), exp2, (dt*u)*B (mul), a*h + b (fma), C*h + y (fma)
OPS_PER_UPDATE = 5
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "scan_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_mamba13b_hbm_traffic.json")


def algorithmic_bytes(x) -> int:
    """Bytes the method must move: u, delta, z read and y written per (b,t,d); B and C
    per (b,t,n); A, D and dt_bias once."""
    esz = 2 if x.io == "bf16" else 4
    per_elem = 4 * esz * x.batch * x.L * x.dim
    bc = 2 * esz * x.batch * x.N * x.L
    params = 4 * (x.A.size + 2 * x.dim)
    return per_elem + bc + params


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(x, rows_batches: int, repeats: int = 3):
    """Time the fp64 oracle on the first ``rows_batches`` batch rows (all channels,
    the full sequence) of the same inputs, with all host threads OpenMP offers;
    ``repeats`` runs, the median is reported."""
    import statistics
    import numpy as np
    import oracle

    nb = min(rows_batches, x.batch)
    sl = slice(0, nb)
    args = [np.ascontiguousarray(a[sl], dtype=np.float64) for a in (x.u, x.delta, x.B, x.C, x.z)]
    A = x.A_dense().astype(np.float64)
    threads = oracle.max_threads()
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.selective_scan_fwd(args[0], args[1], A, args[2], args[3], x.D, args[4], x.dt_bias, nthreads=threads)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    updates = nb * x.L * x.dim * x.N
    return {"value": updates / dt, "unit": "state updates/s", "cores": threads, "kind": "oracle",
            "sample": f"batch rows 0..{nb - 1} of {x.batch} (all {x.dim} channels, full L={x.L}, N={x.N}); "
                      f"{updates:.3e} updates, median of {repeats} runs {dt:.2f} s wall on {threads} OpenMP "
                      f"threads (about {dt * threads * repeats:.0f} s of CPU time in all), fp64"}


PROFILE_COMMANDS = {
    "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/stats -o scan -- python3 bench.py",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {d}/fetch -o scan -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-backward --no-decode --no-ssd",
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {d}/write -o scan -- "
             "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-backward --no-decode --no-ssd",
    "conv_stats": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/convstats -o conv -- "
                  "python3 bench.py --steps 200 --warmup 50 --no-cpu-baseline --no-backward --no-decode --no-ssd --fused-conv",
    "copyfetch": "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {d}/copyfetch -o copy -- "
                 "python3 bench.py --calibrate-copy",
    "copywrite": "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {d}/copywrite -o copy -- "
                 "python3 bench.py --calibrate-copy",
}
COPY_BYTES = 2 << 30
# output directory the profile commands write to (relative to the repository root)
PROFILE_DIR = "rocprof_out"


def calibrate_copy():
    """A plain device-to-device copy of 2 GiB (2 GiB read, 2 GiB written), repeated,
    so that HBM byte counters can be scaled by what they read for known traffic."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_each_way": COPY_BYTES, "launches": 4}))


def summarize_profiles(d):
    """Write profiles/scan_fwd_mamba13b_*.{md,json} from the rocprofv3 CSV outputs
    of PROFILE_COMMANDS run under directory d."""
    import csv
    import statistics

    def counter(sub, prefix, kernel):
        path = os.path.join(d, sub, f"{prefix}_counter_collection.csv")
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if kernel in r["Kernel_Name"]]

    from selective_state_space_79_amd.inputs import make_workload
    x = make_workload(3)
    alg = algorithmic_bytes(x)
    esz = 2
    alg_read = 3 * esz * x.batch * x.L * x.dim + 2 * esz * x.batch * x.N * x.L + 4 * (x.A.size + 2 * x.dim)
    alg_write = esz * x.batch * x.L * x.dim
    fetch = counter("fetch", "scan", "scan_fwd_kernel")
    write = counter("write", "scan", "scan_fwd_kernel")
    cfetch = [v for v in counter("copyfetch", "copy", "") if v > 1e5]
    cwrite = [v for v in counter("copywrite", "copy", "") if v > 1e5]
    kib = COPY_BYTES / 1024
    ffac = kib / statistics.median(cfetch)
    wfac = kib / statistics.median(cwrite)
    rd = statistics.median(fetch) * 1024 * ffac
    wr = statistics.median(write) * 1024 * wfac
    rec = {"kernel": "scan_fwd_kernel<bf16, 4 states/lane, diagonal A, full, 16-byte rows, 4 waves>",
           "workload": "mamba-1.3b-layer (4, 4096, 4096, 16) bf16", "kernel_source_sha256_16": kernel_hash(),
           "fetch_size_kib_per_dispatch": fetch, "write_size_kib_per_dispatch": write,
           "copy_fetch_kib": cfetch, "copy_write_kib": cwrite, "copy_bytes_each_way": COPY_BYTES,
           "fetch_scale": ffac, "write_scale": wfac, "hbm_read_bytes_per_launch": rd,
           "hbm_write_bytes_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
           "algorithmic_read_bytes": alg_read, "algorithmic_write_bytes": alg_write, "algorithmic_bytes": alg,
           "commands": [PROFILE_COMMANDS[k].format(d=PROFILE_DIR) for k in ("fetch", "write", "copyfetch", "copywrite")]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    stats_path = os.path.join(d, "stats", "scan_kernel_stats.csv")
    rows = list(csv.DictReader(open(stats_path)))
    md = ["# scan_fwd_kernel, mamba-1.3b-layer workload (4 x 4096 x 4096, N=16, bf16): rocprofv3 summaries", "",
          f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
          "## Kernel time (`--kernel-trace --stats`)", "",
          "Command (from the repository root on the GPU box):", "",
          "    " + PROFILE_COMMANDS["stats"].format(d=PROFILE_DIR), "",
          "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    md += ["", "## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, one run each)", "",
           "Commands:", ""] + ["    " + c for c in rec["commands"]] + [
           "", "Calibration: a plain 2 GiB device copy (`bench.py --calibrate-copy`) reads "
           f"{statistics.median(cfetch):.0f} KiB of FETCH_SIZE and {statistics.median(cwrite):.0f} KiB of WRITE_SIZE per "
           f"launch for {kib:.0f} KiB moved each way: scale factors {ffac:.4f} (fetch) and {wfac:.4f} (write).", "",
           "| per launch | counter (KiB, median) | scaled bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|",
           f"| read | {statistics.median(fetch):.0f} | {rd:.4g} | {alg_read:.4g} | {rd / alg_read:.3f} |",
           f"| write | {statistics.median(write):.0f} | {wr:.4g} | {alg_write:.4g} | {wr / alg_write:.3f} |",
           f"| total | | {rd + wr:.4g} | {alg:.4g} | {(rd + wr) / alg:.3f} |", ""]
    with open(os.path.join(ROOT, "profiles", "scan_fwd_mamba13b.md"), "w") as f:
        f.write("\n".join(md))
    print(json.dumps({"traffic_bytes_per_launch": rd + wr, "ratio_to_algorithmic": (rd + wr) / alg}))
    conv_stats = os.path.join(d, "convstats", "conv_kernel_stats.csv")
    if os.path.exists(conv_stats):
        rows = list(csv.DictReader(open(conv_stats)))
        md = ["# Fused convolution front end + scan, mamba-1.3b-layer workload (4 x 4096 x 4096, N=16, bf16, "
              "width-4 SiLU convolution): rocprofv3 summary", "",
              f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
              "The run times the plain scan first (`--steps` calls) and then the fused front end (100 calls of "
              "`ssm_selective_scan_fwd_conv`, then the fused decode step); both scans launch the same kernel, so "
              "its calls here are the two kinds together.", "",
              "Command (from the repository root on the GPU box):", "",
              "    " + PROFILE_COMMANDS["conv_stats"].format(d=PROFILE_DIR), "",
              "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
        for r in rows:
            md.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
        with open(os.path.join(ROOT, "profiles", "scan_fwd_conv_mamba13b.md"), "w") as f:
            f.write("\n".join(md) + "\n")
    scalar = re.compile(r"scan_fwd_kernel<[^,]+, \d+, true")
    rows = [r for r in csv.DictReader(open(stats_path))
            if "ssd_" in r["Name"] or scalar.search(r["Name"]) or "scan_carry_kernel" in r["Name"]]
    if any("ssd_" in r["Name"] for r in rows):
        src = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "ssd_fwd.hip")
        with open(src, "rb") as f:
            ssd_hash = hashlib.sha256(f.read()).hexdigest()[:16]
        md = ["# ssd_state_kernel + ssd_out_kernel, scalar-decay large-state workload with one step size per head "
              "(batch 2, L 8192, 64 heads x 64, N 128, bf16): rocprofv3 summary", "",
              f"Kernel source (`csrc/ssd_fwd.hip`) sha256[:16]: `{ssd_hash}`", "",
              "From the same `--kernel-trace --stats` run of the default bench as `scan_fwd_mamba13b.md`; one "
              "`ssm_ssd_fwd` call launches `ssd_state_kernel` (end states of all segments but the last) and then "
              "`ssd_out_kernel`.  The scalar-decay rows of `scan_fwd_kernel` are the per-channel scan timed on the "
              "same inputs for comparison.", "",
              "Command (from the repository root on the GPU box):", "",
              "    " + PROFILE_COMMANDS["stats"].format(d=PROFILE_DIR), "",
              "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
        for r in rows:
            md.append(f"| `{r['Name'][:120]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
        with open(os.path.join(ROOT, "profiles", "ssd_fwd_scalar_decay_head_dt.md"), "w") as f:
            f.write("\n".join(md) + "\n")


def decode_step_bench(batch: int, steps: int = 200, warmup: int = 50):
    """Time ssm_selective_scan_step on a Mamba-1.3B layer (dim 4096, N 16, bf16 I/O,
    fp32 state) decoding `batch` sequences at once: one call = one token each."""
    import numpy as np
    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import make_inputs, to_device

    dim, N = 4096, 16
    x = make_inputs(batch, 1, dim, N, seed=33, io="bf16")
    dev = to_device(x, "cuda:0")
    col = {k: dev[k][..., 0].contiguous() for k in ("u", "delta", "z", "B", "C")}
    rng = np.random.default_rng(34)
    h = torch.from_numpy(rng.standard_normal((batch, dim, N)).astype(np.float32)).cuda()
    y = torch.empty_like(col["u"])
    dims = ssm.make_dims(batch, 1, dim, N, io_dtype=ssm.SSM_BF16)
    stream = torch.cuda.current_stream()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = (p(col["u"]), p(col["delta"]), p(dev["A"]), p(col["B"]), p(col["C"]), p(dev["D"]), p(col["z"]),
            p(dev["dt_bias"]), p(h), p(y), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream))
    fn = ssm.load_library().ssm_selective_scan_step
    for _ in range(warmup):
        assert fn(*args) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn(*args)
    e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # algorithmic bytes: state read + written, A once, u/delta/z read and y written,
    # B and C per sequence, D and dt_bias once
    nbytes = 8 * batch * dim * N + 4 * dim * N + 8 * batch * dim + 4 * batch * N + 8 * dim
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"mamba-1.3b-layer decode step, {batch} sequences (dim {dim}, N {N}, bf16 I/O, fp32 state)",
            "us_per_step": round(us, 3), "tokens_per_s": round(batch / (us * 1e-6), 1),
            "updates_per_s": batch * dim * N / (us * 1e-6), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}


def fused_conv_bench(x, dev, width: int = 4, steps: int = 100, warmup: int = 30):
    """Time ssm_selective_scan_fwd_conv on the same inputs (u taken as the
    convolution's input x, a width-`width` SiLU front end, u not written out) and the
    fused decode step (convolution history + scan state updated in place)."""
    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import io_to_device, make_conv, make_inputs

    w, bb, _ = make_conv(x, width, seed=62)
    wt, bt = torch.from_numpy(w).cuda(), torch.from_numpy(bb).cuda()
    conv = ssm.SsmConv(wt.data_ptr(), bt.data_ptr(), width, 1)
    y = torch.empty_like(dev["u"])
    dims = ssm.dims_for(dev["u"], dev["B"], dev["A"])
    stream = torch.cuda.current_stream()
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    args = (p(dev["u"]), ctypes.byref(conv), None, p(dev["delta"]), p(dev["A"]), p(dev["B"]), p(dev["C"]),
            p(dev["D"]), p(dev["z"]), p(dev["dt_bias"]), None, None, p(y), None, ctypes.byref(dims),
            ctypes.c_void_p(stream.cuda_stream))
    fn = ssm.load_library().ssm_selective_scan_fwd_conv

    def timed(call, n, nw):
        for _ in range(nw):
            st = call()
            if st != 0:
                raise ssm.SsmError(st, "fused conv")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(lambda: fn(*args), steps, warmup)
    nbytes = algorithmic_bytes(x) + 4 * x.dim * (width + 1)
    out = {"workload": f"{x.batch}x{x.L}x{x.dim}, N {x.N}, {x.io} I/O, width-{width} SiLU front end fused",
           "ms_per_call": round(ms, 4), "updates_per_s": x.updates / (ms * 1e-3),
           "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": nbytes}
    decode = []
    for batch in (64, 256):
        xd = make_inputs(batch, 1, x.dim, x.N, seed=63, io=x.io)
        dd = {k: v for k, v in to_device_cols(xd).items()}
        wd, bd, st = make_conv(xd, width, seed=64, with_state=True)
        cst = io_to_device(xd, st)
        h = torch.zeros((batch, x.dim, x.N), dtype=torch.float32, device="cuda:0")
        yd = torch.empty_like(dd["u"])
        wdt, bdt = torch.from_numpy(wd).cuda(), torch.from_numpy(bd).cuda()
        cv = ssm.SsmConv(wdt.data_ptr(), bdt.data_ptr(), width, 1)
        sd = ssm.make_dims(batch, 1, x.dim, x.N, io_dtype=ssm.SSM_BF16 if x.io == "bf16" else ssm.SSM_F32)
        a2 = (p(dd["u"]), ctypes.byref(cv), p(cst), p(dd["delta"]), p(dev["A"]), p(dd["B"]), p(dd["C"]), p(dev["D"]),
              p(dd["z"]), p(dev["dt_bias"]), p(h), None, p(yd), ctypes.byref(sd), ctypes.c_void_p(stream.cuda_stream))
        f2 = ssm.load_library().ssm_selective_scan_step_conv
        us = timed(lambda: f2(*a2), 200, 50) * 1e3
        esz = 2 if x.io == "bf16" else 4
        # state read and written; A; x, delta, z read and y written; B, C; D, dt_bias;
        # the convolution history read and written; its weights and bias
        nb = (8 * batch * x.dim * x.N + 4 * x.dim * x.N + 4 * esz * batch * x.dim + 2 * esz * batch * x.N
              + 8 * x.dim + 2 * esz * batch * x.dim * (width - 1) + 4 * x.dim * (width + 1))
        decode.append({"sequences": batch, "us_per_step": round(us, 3), "tokens_per_s": round(batch / (us * 1e-6), 1),
                       "gbs": round(nb / (us * 1e-6) / 1e9, 1), "hbm_frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "algorithmic_bytes": nb})
    out["decode_step"] = decode
    return out


def to_device_cols(xd):
    """Device tensors of a one-token input set, the token axis dropped: (batch, dim)
    and (batch, N)."""
    from selective_state_space_79_amd.inputs import to_device

    dev = to_device(xd, "cuda:0")
    return {k: (dev[k][..., 0].contiguous() if k in ("u", "delta", "z", "B", "C") else dev[k]) for k in dev}


# minimal VALU operations per state update of the backward pass: the forward recompute
# with its read-out (mul, exp2, mul, fma, fma), the reverse step (g = ds*C + e: fma;
# e = a*g: mul; a*h_prev: mul; g*(a*h_prev): mul; dA, sum A*.., sum g*B: 3 fma;
# ds*h and g*x for dC, dB: 2 mul) and the sums of dB and dC over channels (2 add)
BWD_OPS_PER_UPDATE = 16


def backward_bench(x, dev, steps: int = 40, warmup: int = 15):
    """Time ssm_selective_scan_bwd on the same inputs (cotangent dy seeded, no dh_last):
    one call = every kernel of the backward (state checkpoints, reverse gradient walk,
    reductions of the partial sums)."""
    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import io_to_device, make_cotangents

    dy = io_to_device(x, make_cotangents(x, seed=53)[0], "cuda:0")
    dims = ssm.dims_for(dev["u"], dev["B"], dev["A"])
    plan = ssm.ssm_selective_scan_bwd_plan(dims).as_dict()
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
    dims.workspace, dims.workspace_bytes = ws.data_ptr(), plan["workspace_bytes"]
    f32 = dict(dtype=torch.float32, device="cuda:0")
    out = {"du": torch.empty_like(dev["u"]), "ddelta": torch.empty_like(dev["u"]), "dz": torch.empty_like(dev["u"]),
           "dA": torch.empty(dev["A"].shape, **f32), "dB": torch.empty((x.batch, x.N, x.L), **f32),
           "dC": torch.empty((x.batch, x.N, x.L), **f32), "dD": torch.empty(x.dim, **f32),
           "ddt_bias": torch.empty(x.dim, **f32), "dh0": None}
    grads = ssm.SsmGrads(*[out[k].data_ptr() if out[k] is not None else None for k, _ in ssm.SsmGrads._fields_])
    stream = torch.cuda.current_stream()
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    args = (p(dev["u"]), p(dev["delta"]), p(dev["A"]), p(dev["B"]), p(dev["C"]), p(dev["D"]), p(dev["z"]),
            p(dev["dt_bias"]), None, p(dy), None, ctypes.byref(grads), ctypes.byref(dims),
            ctypes.c_void_p(stream.cuda_stream))
    fn = ssm.load_library().ssm_selective_scan_bwd
    for _ in range(warmup):
        st = fn(*args)
        if st != 0:
            raise ssm.SsmError(st, "ssm_selective_scan_bwd")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn(*args)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    esz = 2 if x.io == "bf16" else 4
    # u, delta, z, dy read and du, ddelta, dz written per element; B, C read and dB, dC
    # (float32) written per (b, t, n); A, D, dt_bias read and dA, dD, ddt_bias written
    nbytes = (7 * esz * x.batch * x.L * x.dim + (2 * esz + 8) * x.batch * x.N * x.L
              + 8 * (x.A.size + 2 * x.dim))
    tops = BWD_OPS_PER_UPDATE * x.updates / (ms * 1e-3) / 1e12
    rec = {"workload": f"{x.batch}x{x.L}x{x.dim}, N {x.N}, {x.io} I/O: gradients of every input",
           "ms_per_call": round(ms, 4), "updates_per_s": x.updates / (ms * 1e-3), "plan": plan,
           "roofline": {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 2),
                        "unit": "TFLOP/s", "frac": round(tops / VALU_PEAK_TOPS, 4),
                        "note": f"{BWD_OPS_PER_UPDATE} fp32 VALU lane operations per state update"},
           "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}

    # training with saved checkpoints: the forward keeps the state every 16 steps and
    # the backward starts from them instead of recomputing them
    nck = ssm.ssm_selective_scan_ckpt_bytes(dims)
    if nck:
        ck = torch.empty(nck // 4, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(dev["u"])
        fargs = (p(dev["u"]), p(dev["delta"]), p(dev["A"]), p(dev["B"]), p(dev["C"]), p(dev["D"]), p(dev["z"]),
                 p(dev["dt_bias"]), None, p(y), None, p(ck), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream))
        bargs = args[:11] + (p(ck),) + args[11:]
        lib = ssm.load_library()

        def timed(fn, a, name):
            for _ in range(warmup):
                st = fn(*a)
                if st != 0:
                    raise ssm.SsmError(st, name)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(steps):
                fn(*a)
            t1.record(stream)
            t1.synchronize()
            return t0.elapsed_time(t1) / steps

        f_ms = timed(lib.ssm_selective_scan_fwd_ckpt, fargs, "ssm_selective_scan_fwd_ckpt")
        b_ms = timed(lib.ssm_selective_scan_bwd_ckpt, bargs, "ssm_selective_scan_bwd_ckpt")
        rec["with_forward_checkpoints"] = {
            "fwd_ckpt_ms": round(f_ms, 4), "bwd_ckpt_ms": round(b_ms, 4), "checkpoint_bytes": nck,
            "note": "ssm_selective_scan_fwd_ckpt keeps the state every 16 steps; ssm_selective_scan_bwd_ckpt "
                    "starts from them and skips its own recomputation walk"}
    return rec


MFMA_BF16_PEAK_TFLOPS = 2500.0


def ssd_bench(steps: int = 100, warmup: int = 30):
    """Time ssm_ssd_fwd, the chunked state-space-duality pass, on the scalar-decay
    large-state workload with one step size per head (batch 2, L 8192, 64 heads x 64
    channels, N 128, bf16 I/O); one call = both of its kernels.  The per-channel scan
    (ssm_selective_scan_fwd in scalar-decay mode) is timed on the same inputs, each
    head's step input repeated over its channels."""
    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import SSD_WORKLOADS, make_ssd_workload, ssd_to_device, to_device

    x = make_ssd_workload()
    d = ssd_to_device(x, "cuda:0")
    y = torch.empty_like(d["u"])
    dims = ssm.make_ssd_dims(x.batch, x.L, x.nheads, x.N, headdim=x.headdim)
    need = ssm.ssm_ssd_fwd_workspace_bytes(dims)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda:0")
    dims.workspace, dims.workspace_bytes = ws.data_ptr(), need
    stream = torch.cuda.current_stream()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    args = (p(d["u"]), p(d["delta"]), p(d["A"]), p(d["B"]), p(d["C"]), p(d["D"]), p(d["z"]), p(d["dt_bias"]), None,
            p(y), None, ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream))
    fn = ssm.load_library().ssm_ssd_fwd

    def timed(call, n, w):
        for _ in range(w):
            st = call()
            if st != 0:
                raise ssm.SsmError(st, "bench call")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            call()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(lambda: fn(*args), steps, warmup)
    # the per-channel scan on the same inputs
    sc = to_device(x.per_channel(), "cuda:0")
    ys = torch.empty_like(sc["u"])
    sdims = ssm.dims_for(sc["u"], sc["B"], sc["A"])
    splan = ssm.ssm_selective_scan_plan(sdims).as_dict()
    sws = torch.empty(max(splan["workspace_bytes"], 1), dtype=torch.uint8, device="cuda:0")
    sdims.workspace, sdims.workspace_bytes = sws.data_ptr(), splan["workspace_bytes"]
    sargs = (p(sc["u"]), p(sc["delta"]), p(sc["A"]), p(sc["B"]), p(sc["C"]), p(sc["D"]), p(sc["z"]),
             p(sc["dt_bias"]), p(ys), ctypes.byref(sdims), ctypes.c_void_p(stream.cuda_stream))
    sfn = ssm.load_library().ssm_selective_scan_fwd
    ms_scan = timed(lambda: sfn(*sargs), max(steps // 5, 5), 3)
    del sc, ys, sws

    # algorithmic bytes: u, z read and y written per (b,t,d); the step input per
    # (b,h,t); B and C per (b,t,n); A, dt_bias per head and D per channel
    nbytes = (3 * 2 * x.batch * x.L * x.dim + 2 * x.batch * x.nheads * x.L + 2 * 2 * x.batch * x.N * x.L
              + 4 * (2 * x.nheads + x.dim))
    gbs = nbytes / (ms * 1e-3) / 1e9
    # matrix work the chunked method issues per head and 64-step chunk: 10 lower-
    # triangular 16x16 tiles of C^T B (N-deep), the masked product (6 16x32 blocks per
    # 16 channels, two bf16 parts), the state read and the state update (N x 64 x 64
    # each, two parts); the end states of all but the last segment repeat the update
    plan = ssm.ssm_ssd_fwd_plan(dims).as_dict()
    nseg = plan["nsegments"]
    chunks = x.batch * x.nheads * -(-x.L // 64)
    mac_chunk = 10 * 256 * x.N + 2 * 4 * 6 * 16 * 16 * 32 + 2 * 64 * 64 * x.N + 2 * x.N * 64 * 64
    mac_state = 2 * x.N * 64 * 64 * (nseg - 1) / nseg
    tflops = 2 * chunks * (mac_chunk + mac_state) / (ms * 1e-3) / 1e12
    return {"workload": f"{SSD_WORKLOADS[5]['name']}: batch {x.batch}, L {x.L}, {x.nheads} heads x {x.headdim}, "
                        f"N {x.N}, bf16 I/O, one step size per head",
            "ms_per_call": round(ms, 4), "updates_per_s": x.updates / (ms * 1e-3), "plan": plan,
            "hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes},
            "mfma": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "note": "bf16 matrix FLOPs the chunked method issues (operands split in two bf16 parts)"},
            "per_channel_scan_same_inputs": {"ms_per_call": round(ms_scan, 4),
                                             "updates_per_s": x.updates / (ms_scan * 1e-3),
                                             "speedup_of_chunked": round(ms_scan / ms, 2)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3, help="1..5; the reported line is workload 3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass timing")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step timing")
    ap.add_argument("--no-ssd", action="store_true",
                    help="skip the chunked scalar-decay (per-head step) pass on the large-state workload")
    ap.add_argument("--fused-conv", action="store_true",
                    help="also time the fused convolution front end (same scan kernel, so off by default: "
                         "its launches would mix into the scan kernel's profile)")
    ap.add_argument("--cpu-batches", type=int, default=4, help="batch rows in the oracle's timing sample")
    ap.add_argument("--calibrate-copy", action="store_true", help="only run a 2 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSVs in DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the library "
              "has no multi-GPU path; the scan is sharded over batch/channels with no communication when it is "
              "run once per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import WORKLOADS, make_workload, to_device

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib = ssm.load_library()
    torch.cuda.set_device(0)
    w = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    x = make_workload(args.workload)
    dev = to_device(x, "cuda:0")
    gen_s = time.perf_counter() - t_gen

    stream = torch.cuda.current_stream()
    y = torch.empty_like(dev["u"])
    dims = ssm.dims_for(dev["u"], dev["B"], dev["A"])
    plan = ssm.ssm_selective_scan_plan(dims).as_dict()
    ws = None
    if plan["workspace_bytes"]:
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
        dims.workspace, dims.workspace_bytes = ws.data_ptr(), plan["workspace_bytes"]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    call_args = (p(dev["u"]), p(dev["delta"]), p(dev["A"]), p(dev["B"]), p(dev["C"]), p(dev["D"]), p(dev["z"]),
                 p(dev["dt_bias"]), p(y), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream))
    fn = lib.ssm_selective_scan_fwd

    def step():
        st = fn(*call_args)
        if st != 0:
            raise ssm.SsmError(st, "ssm_selective_scan_fwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    # barrier + synchronize on both sides (one process: the barrier is trivial)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    ev1.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_events = ev0.elapsed_time(ev1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    ms_per_step = max(ms_events, ms_wall)

    updates = x.updates
    value = updates / (ms_per_step * 1e-3)
    nbytes = algorithmic_bytes(x)
    # the dominant kernel: with one piece per sequence a step is one launch of it
    kernel_ms = ms_events
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    tops = OPS_PER_UPDATE * updates / (kernel_ms * 1e-3) / 1e12
    traffic = measured_traffic() if (args.workload == 3 and plan["nchunks"] == 1) else None
    alu = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TFLOP/s",
           "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
           "note": "FLOP = one fp32 VALU lane operation; 5 per state update (mul, exp2, mul, fma, fma); peak = "
                   "256 CU x 64 lanes x 2.4 GHz, packed fp32 not used"}
    hbm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
           "algorithmic_bytes_per_launch": nbytes}
    roofline = alu if alu["frac"] >= hbm["frac"] else hbm

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "state updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w["name"], "batch": x.batch, "seqlen": x.L, "dim": x.dim, "dstate": x.N,
                   "nheads": x.nheads, "io_dtype": x.io, "state_dtype": "f32", "seed": args.workload,
                   "plan": plan},
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "hbm": hbm,
        "timing": {"ms_events": ms_events, "ms_wall": ms_wall, "input_gen_s": round(gen_s, 2),
                   "kernel_source_sha256_16": kernel_hash(), "device": torch.cuda.get_device_name(0)},
    }
    if args.workload == 3 and not args.no_decode:
        rec["decode_step"] = [decode_step_bench(64), decode_step_bench(256)]
    if args.fused_conv:
        rec["fused_conv"] = fused_conv_bench(x, dev)
    if not args.no_backward:
        rec["backward"] = backward_bench(x, dev)
    if not args.no_ssd:
        del dev, y
        torch.cuda.empty_cache()
        rec["ssd"] = ssd_bench()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_batches)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
