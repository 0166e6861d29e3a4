#!/usr/bin/env python3
"""Benchmark of the selective-scan forward pass on one MI355X.

One step = one call of ssm_selective_scan_fwd over the whole Mamba-1.3B-shaped
layer workload (batch 4, L 4096, dim 4096, dstate 16, bf16 I/O, fp32 state):
every stage of the path (loads, softplus, discretisation, scan, read-out, skip,
gate, bf16 store) runs inside the timed region, with inputs already in HBM.

Prints one JSON line.  ``value`` is state updates per second (B*L*D*N / step time);
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


def measured_traffic(launch_units: float):
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


def cpu_baseline(x, rows_batches: int):
    """Time the fp64 oracle on the first ``rows_batches`` batch rows (all channels,
    the full sequence) of the same inputs, with all host threads OpenMP offers."""
    import numpy as np
    import oracle

    nb = min(rows_batches, x.batch)
    sl = slice(0, nb)
    args = [np.ascontiguousarray(a[sl], dtype=np.float64) for a in (x.u, x.delta, x.B, x.C, x.z)]
    A = x.A_dense().astype(np.float64)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.selective_scan_fwd(args[0], args[1], A, args[2], args[3], x.D, args[4], x.dt_bias, nthreads=threads)
    dt = time.perf_counter() - t0
    updates = nb * x.L * x.dim * x.N
    return {"value": updates / dt, "unit": "state updates/s", "cores": threads, "kind": "oracle",
            "sample": f"batch rows 0..{nb - 1} of {x.batch} (all {x.dim} channels, full L={x.L}, N={x.N}); "
                      f"{updates:.3e} updates in {dt:.2f} s wall on {threads} OpenMP threads, fp64"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, help="1..5; the reported line is workload 3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-batches", type=int, default=2, help="batch rows in the oracle's timing sample")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this build "
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
    traffic = measured_traffic(1.0) if (args.workload == 3 and plan["nchunks"] == 1) else None
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
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_batches)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
