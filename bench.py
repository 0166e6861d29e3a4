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
# scalar decay (one rate per head): the decay is one exp2 per (b,t,d), shared by the
# state entries; per update x*B (mul), a*h + b (fma), C*h + y (fma)
OPS_PER_UPDATE_SCALAR = 3
KERNEL_SRC = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "scan_fwd.hip")
CHUNKED_SRC = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "scan_chunked.hip")
CHUNKED_FILE = os.path.join(ROOT, "profiles", "scan_chunked_scalar_decay_counters.json")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_mamba13b_hbm_traffic.json")
VALU_FILE = os.path.join(ROOT, "profiles", "scan_fwd_mamba13b_valu_issue.json")
SIMDS = 256 * 4
MFMA_BF16_PEAK_TFLOPS = 2500.0
CLOCK_HZ = 2.4e9

# Untimed warm-up runs for at least this long, whatever --warmup asks for: the GPU clock
# ramps up over the first milliseconds of work, and a handful of 0.3 ms calls would
# otherwise time the ramp.  The number of warm-up calls actually run is reported.
MIN_WARMUP_S = 0.25


def time_calls(call, steps: int, warmup: int, stream, min_warmup_s: float | None = None):
    """Warm up with at least `warmup` calls and at least `min_warmup_s` seconds, then
    time exactly `steps` calls bracketed by two HIP events recorded on `stream` (the
    stream the kernels are launched on) and by the wall clock, with a device
    synchronisation on both sides: the mean per call (`ms_events`, `ms_wall`,
    `ms_per_step` = the larger).  Then the same number of calls again, each bracketed by
    its own pair of events, for the distribution (median, min, max, p90); an event
    between two launches costs short kernels a few microseconds, so the mean is taken
    from the first loop only.  call(i) launches call number i (i lets the caller rotate
    input sets).  Returns the statistics in milliseconds."""
    import statistics
    import torch

    if min_warmup_s is None:
        min_warmup_s = MIN_WARMUP_S
    n = 0
    t0 = time.perf_counter()
    while n < warmup or time.perf_counter() - t0 < min_warmup_s:
        call(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()   # keep the host within a few calls of the device
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        call(i)
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total = e0.elapsed_time(e1)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record(stream)
        call(i)
        ev[2 * i + 1].record(stream)
    ev[-1].synchronize()
    per = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    return {"ms_events": total / steps, "ms_wall": wall * 1e3 / steps, "ms_per_step": max(total / steps, wall * 1e3 / steps),
            "ms_median": statistics.median(per), "ms_min": per[0], "ms_max": per[-1],
            "ms_p90": per[min(len(per) - 1, int(0.9 * len(per)))], "warmup_calls_run": n,
            "warmup_s": round(warm_s, 3)}


def algorithmic_bytes(x) -> int:
    """Bytes the method must move: u, delta, z read and y written per (b,t,d); B and C
    per (b,t,n); A, D and dt_bias once."""
    esz = 2 if x.io == "bf16" else 4
    per_elem = 4 * esz * x.batch * x.L * x.dim
    bc = 2 * esz * x.batch * x.N * x.L
    params = 4 * (x.A.size + 2 * x.dim)
    return per_elem + bc + params


# Inputs of a workload smaller than this are rotated over several resident copies, so
# that the 256 MB Infinity Cache cannot serve a call from the previous call's data.
ROTATE_BYTES = 512 << 20


def scan_workload_bench(x, dev, steps: int, warmup: int, stream, extra_sets=None):
    """Time ssm_selective_scan_fwd over the workload x (device tensors `dev`; further
    input sets `extra_sets` are rotated call by call).  One call = the whole forward
    pass of the workload, every kernel it launches.  Returns its record: plan, timing
    statistics, updates/s and both rooflines of the call (algorithmic bytes against the
    HBM peak; fp32 VALU lane operations against the VALU peak)."""
    import torch
    import selective_state_space_79_amd as ssm

    sets = [dev] + list(extra_sets or [])
    dims = ssm.dims_for(dev["u"], dev["B"], dev["A"])
    plan = ssm.ssm_selective_scan_plan(dims).as_dict()
    ws = None
    if plan["workspace_bytes"]:
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda:0")
        dims.workspace, dims.workspace_bytes = ws.data_ptr(), plan["workspace_bytes"]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    ys = [torch.empty_like(d["u"]) for d in sets]
    argsets = [(p(d["u"]), p(d["delta"]), p(d["A"]), p(d["B"]), p(d["C"]), p(d["D"]), p(d["z"]), p(d["dt_bias"]),
                p(y), ctypes.byref(dims), ctypes.c_void_p(stream.cuda_stream)) for d, y in zip(sets, ys)]
    fn = ssm.load_library().ssm_selective_scan_fwd

    def call(i):
        st = fn(*argsets[i % len(argsets)])
        if st != 0:
            raise ssm.SsmError(st, "ssm_selective_scan_fwd")

    t = time_calls(call, steps, warmup, stream)
    ms = t["ms_events"]            # average call duration, HIP events on the launch stream
    nbytes = algorithmic_bytes(x)
    gbs = nbytes / (ms * 1e-3) / 1e9
    scalar = x.nheads > 0
    ops = OPS_PER_UPDATE_SCALAR if scalar else OPS_PER_UPDATE
    tops = ops * x.updates / (ms * 1e-3) / 1e12
    ceiling = ops / (ops + (0 if scalar else 1))   # the exp2 is half rate (diagonal A only)
    alu = {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TFLOP/s",
           "frac": round(tops / VALU_PEAK_TOPS, 4), "traffic": None,
           "note": (f"FLOP = one fp32 VALU lane operation; {ops} per state update ("
                    + ("x*B mul, a*h+b fma, C*h+y fma; the decay's exp2 is per (b,t,d)" if scalar else
                       "dt*A mul, exp2, x*B mul, a*h+b fma, C*h+y fma")
                    + "); peak = 256 CU x 64 lanes x 2.4 GHz, packed fp32 not used"
                    + ("" if scalar else "; v_exp_f32 issues at half rate, so 6 issue slots carry these 5 "
                       "operations and frac cannot exceed 5/6 = 0.833")),
           "frac_ceiling": round(ceiling, 4)}
    hbm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes_per_launch": nbytes}
    rec = {"workload": f"{x.batch}x{x.L}x{x.dim}, N {x.N}, {x.io} I/O" + (f", {x.nheads} heads scalar decay"
                                                                       if scalar else ", diagonal A"),
           "plan": plan, "timing": t, "ms_per_call": round(t["ms_per_step"], 5),
           "updates_per_s": x.updates / (t["ms_per_step"] * 1e-3), "gbs": round(gbs, 1),
           "input_sets_rotated": len(sets), "hbm": hbm, "alu": alu,
           "roofline": alu if alu["frac"] >= hbm["frac"] else hbm}
    if plan.get("form") == 1:
        # the chunked form does not walk the recurrence (3 operations per state update):
        # its contractions over the state are matrix products, so it is measured against
        # the matrix-core and HBM roofs, and its VALU issue comes from the counters
        del rec["alu"]
        mf = chunked_mfma_flops(x, plan)
        tf = mf / (ms * 1e-3) / 1e12
        mfma = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None, "flops_per_call": mf,
                "note": "bf16 matrix work the chunked form issues (fp32 operands split in two bf16 parts count "
                        "twice): C^T B per 16-step chunk in each of a workgroup's 4 waves, the state read and the "
                        "state update per chunk, and the piece aggregate of all pieces but the last"}
        rec["form"] = "chunked: state read, state update and C^T B on the matrix cores per 16-step chunk"
        rec["mfma"] = mfma
        rec["roofline"] = mfma if mfma["frac"] >= hbm["frac"] else hbm
        vi = measured_chunked_issue(x, ms)
        if vi:
            rec["valu_issue"] = vi
    if plan["nchunks"] == 1 and not scalar:
        vi = measured_valu_issue(x, ms)
        if vi:
            rec["valu_issue"] = vi
    return rec


def other_workloads_bench(indices, steps: int, warmup: int, stream):
    """scan_workload_bench on the other named workloads, one at a time (inputs freed
    in between); a workload smaller than ROTATE_BYTES is rotated over copies drawn from
    further seeds."""
    import torch
    from selective_state_space_79_amd.inputs import WORKLOADS, make_workload, to_device

    out = {}
    for idx in indices:
        x = make_workload(idx)
        dev = to_device(x, "cuda:0")
        nsets = 1
        if algorithmic_bytes(x) < ROTATE_BYTES and x.updates > 1e6:
            nsets = -(-ROTATE_BYTES // algorithmic_bytes(x))
        extra = [to_device(make_workload(idx, seed=1000 + 17 * k + idx), "cuda:0") for k in range(1, nsets)]
        r = scan_workload_bench(x, dev, steps, warmup, stream, extra_sets=extra)
        r["seed"] = idx
        out[WORKLOADS[idx]["name"]] = r
        progress(f"workload {idx} timed: {r['ms_per_call']:.4f} ms per call")
        del dev, extra, x
        torch.cuda.empty_cache()
    return out


def linear_in_L_bench(steps: int, warmup: int, stream, Ls=(1024, 2048, 4096, 8192)):
    """Call time of a 1.3B-layer-like shape (batch 5, dim 4096, N 16, bf16) at several
    sequence lengths, the same plan (one piece, 320 workgroups) at each: the scan's
    work is linear in L, so the time should be too.  (Batch 5 rather than 4 gives these
    launches a grid of their own, so a profile tells them apart from the headline's.)"""
    import numpy as np
    from selective_state_space_79_amd.inputs import ScanInputs, make_inputs, to_device

    big = make_inputs(5, max(Ls), 4096, 16, seed=77, io="bf16")
    rows = []
    for L in Ls:
        cut = lambda a: np.ascontiguousarray(a[..., :L])
        x = ScanInputs(big.batch, L, big.dim, big.N, 0, "bf16", cut(big.u), cut(big.delta), cut(big.z), cut(big.B),
                       cut(big.C), big.A, big.D, big.dt_bias)
        r = scan_workload_bench(x, to_device(x, "cuda:0"), steps, warmup, stream)
        rows.append({"L": L, "ms_median": round(r["timing"]["ms_median"], 5), "ms_mean": round(r["timing"]["ms_events"], 5),
                     "updates_per_s": r["updates_per_s"], "workgroups": r["plan"]["workgroups"]})
    base = rows[0]
    for r in rows:
        r["time_ratio_to_first"] = round(r["ms_median"] / base["ms_median"], 3)
        r["L_ratio_to_first"] = r["L"] / base["L"]
    return rows


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


def measured_valu_issue(x, ms):
    """VALU issue occupancy of the forward kernel from the committed rocprofv3 counters
    (SQ_INSTS_VALU and SQ_INSTS_VALU_TRANS_F32 per dispatch), if they were taken on the
    current kernel source and this workload's shape; else None.  A wave64 VALU
    instruction holds a SIMD16 for 4 cycles, a transcendental one for 8, so the issue
    cycles are 4 x (VALU + TRANS); the fraction is over 1024 SIMDs x 2.4 GHz x the call
    time measured here."""
    try:
        with open(VALU_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_hash():
        return None
    if rec.get("shape") != [x.batch, x.L, x.dim, x.N]:
        return None
    v, tr = rec["SQ_INSTS_VALU"], rec["SQ_INSTS_VALU_TRANS_F32"]
    cycles = 4 * (v + tr)
    avail = SIMDS * CLOCK_HZ * ms * 1e-3
    # the method's own floor: 6 issue slots per state update (5 operations, exp2 at half
    # rate), wave64 instructions
    walk = 4 * 6 * x.updates / 64
    return {"valu_instructions_per_call": v, "trans_instructions_per_call": tr, "issue_cycles_per_call": cycles,
            "issue_frac": round(cycles / avail, 4), "walk_floor_issue_frac": round(walk / avail, 4),
            "issue_cycles_over_walk_floor": round(cycles / walk, 3),
            "note": "issue_frac = 4*(VALU+TRANS) cycles / (1024 SIMDs x 2.4 GHz x call time); walk floor = 6 slots "
                    "per state update; counters from " + os.path.relpath(VALU_FILE, ROOT)}


def chunked_hash() -> str:
    with open(CHUNKED_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def chunked_mfma_flops(x, plan) -> float:
    """bf16 matrix flops one call of the chunked form issues (split operands twice):
    per 64-channel block and 16-step chunk, C^T B (16 x 16, depth N) in each of the 4
    waves, the state read (16 x 64, depth N, two parts) and the state update (N x 64,
    depth 16, two parts); the matrix-core piece aggregate adds N x 64 depth-1 products
    in two parts per step of every piece but the last."""
    import math

    blocks = x.batch * math.ceil(x.dim / 64)
    chunks = math.ceil(x.L / 16)
    per = 4 * 2 * 16 * 16 * x.N + 2 * 2 * 16 * 64 * x.N + 2 * 2 * x.N * 64 * 16
    agg_steps = min(x.L, (plan["nchunks"] - 1) * plan["chunk_len"])
    return float(blocks * chunks * per + blocks * agg_steps * 2 * 2 * x.N * 64)


def measured_chunked_issue(x, ms):
    """VALU issue of the chunked form's kernels (piece aggregate, carry, chunked pass)
    from the committed rocprofv3 counters, if they were taken on the current source and
    this shape; else None."""
    try:
        with open(CHUNKED_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != chunked_hash() or rec.get("shape") != [x.batch, x.L, x.dim, x.N]:
        return None
    v, tr = rec["SQ_INSTS_VALU"], rec["SQ_INSTS_VALU_TRANS_F32"]
    cycles = 4 * (v + tr)
    avail = SIMDS * CLOCK_HZ * ms * 1e-3
    return {"valu_instructions_per_call": v, "trans_instructions_per_call": tr, "issue_cycles_per_call": cycles,
            "issue_frac": round(cycles / avail, 4),
            "note": "issue_frac = 4*(VALU+TRANS) cycles of the call's kernels / (1024 SIMDs x 2.4 GHz x call time); "
                    "counters from " + os.path.relpath(CHUNKED_FILE, ROOT)}


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
    # one thread, on the first 256 channels of batch row 0 (full L)
    nd = min(256, x.dim)
    one = [np.ascontiguousarray(a[0:1, 0:nd], dtype=np.float64) for a in (x.u, x.delta, x.z)]
    t1 = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.selective_scan_fwd(one[0], one[1], A[:nd], args[2][0:1], args[3][0:1], x.D[:nd], one[2],
                                  x.dt_bias[:nd], nthreads=1)
        t1.append(time.perf_counter() - t0)
    dt1 = statistics.median(t1)
    up1 = x.L * nd * x.N
    return {"value": updates / dt, "unit": "state updates/s", "cores": threads, "kind": "oracle",
            "sample": f"batch rows 0..{nb - 1} of {x.batch} (all {x.dim} channels, full L={x.L}, N={x.N}); "
                      f"{updates:.3e} updates, median of {repeats} runs {dt:.2f} s wall on {threads} OpenMP "
                      f"threads (about {dt * threads * repeats:.0f} s of CPU time in all), fp64",
            "single_thread": {"value": up1 / dt1, "unit": "state updates/s", "cores": 1,
                              "sample": f"batch row 0, channels 0..{nd - 1}, full L={x.L}, N={x.N}: {up1:.3e} "
                                        f"updates, median of {repeats} runs {dt1:.2f} s, fp64"}}


# the counter passes time only the headline workload, with no warm-up floor (every
# dispatch is serialised and sampled under --pmc)
_ONLY = "--steps 3 --warmup 1 --min-warmup-s 0 --no-cpu-baseline --no-backward --no-decode --no-ssd --no-workloads --no-linear"
PROFILE_COMMANDS = {
    "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/stats -o scan -- python3 bench.py",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {d}/fetch -o scan -- python3 bench.py " + _ONLY,
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {d}/write -o scan -- python3 bench.py " + _ONLY,
    "valu": "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS SQ_INSTS_SALU SQ_BUSY_CYCLES "
            "--kernel-trace --output-format csv -d {d}/valu -o scan -- python3 bench.py --steps 3 --warmup 1 "
            "--min-warmup-s 0 --no-cpu-baseline --no-decode --no-ssd --no-workloads --no-linear",
    "conv_stats": "rocprofv3 --kernel-trace --stats --output-format csv -d {d}/convstats -o conv -- "
                  "python3 bench.py --steps 200 --warmup 50 --no-cpu-baseline --no-backward --no-decode --no-ssd "
                  "--no-workloads --no-linear --fused-conv",
    "copyfetch": "rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d {d}/copyfetch -o copy -- "
                 "python3 bench.py --calibrate-copy",
    "copywrite": "rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d {d}/copywrite -o copy -- "
                 "python3 bench.py --calibrate-copy",
    "bwd_counters": "rocprofv3 --kernel-include-regex scan_bwd_ --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
                    "SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_SALU "
                    "GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d {d}/bwdctr -o scan -- python3 bench.py "
                    "--steps 3 --warmup 1 --min-warmup-s 0 --no-cpu-baseline --no-decode --no-ssd --no-workloads "
                    "--no-linear",
    "chunked_counters": "rocprofv3 --kernel-include-regex 'scan_chunked|scan_piece_states|scan_carry' --pmc SQ_WAVES "
                        "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
                        "SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS GRBM_GUI_ACTIVE --kernel-trace --output-format csv "
                        "-d {d}/chkctr -o scan -- python3 bench.py --steps 3 --warmup 1 --min-warmup-s 0 "
                        "--no-cpu-baseline --no-backward --no-decode --no-ssd --no-linear --only-workloads 5",
    "ssd_counters": "rocprofv3 --kernel-include-regex ssd_ --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
                    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
                    "GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d {d}/ssdctr -o scan -- python3 bench.py "
                    "--steps 3 --warmup 1 --min-warmup-s 0 --no-cpu-baseline --no-backward --no-decode --no-workloads "
                    "--no-linear",
}
COPY_BYTES = 2 << 30
# output directory the profile commands write to (relative to the repository root); raw
# rocprofv3 output stays out of the repository's tracked files
PROFILE_DIR = "gpurun_out/rocprof"


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


def _grid(row) -> int:
    """Work-items of a dispatch from a rocprofv3 CSV row (Grid_Size, or its x/y/z)."""
    if row.get("Grid_Size"):
        return int(float(row["Grid_Size"]))
    g = 1
    for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"):
        if row.get(k):
            g *= int(float(row[k]))
    return g


def _trace_rows(path):
    """Per (kernel, grid) dispatch statistics from a rocprofv3 kernel_trace.csv, in ns:
    calls, average, median, min, max, ordered by total time."""
    import csv
    import statistics

    by = {}
    for r in csv.DictReader(open(path)):
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by.setdefault((r["Kernel_Name"], _grid(r)), []).append(ns)
    rows = [{"name": k[0], "grid": k[1], "calls": len(v), "avg": statistics.fmean(v), "median": statistics.median(v),
             "min": min(v), "max": max(v), "total": sum(v)} for k, v in by.items()]
    return sorted(rows, key=lambda r: -r["total"])


def _trace_table(rows, width=110):
    md = ["| kernel | grid (work-items) | calls | average ns | median ns | min ns | max ns |",
          "|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| `{r['name'][:width]}` | {r['grid']} | {r['calls']} | {r['avg']:.0f} | {r['median']:.0f} | "
                  f"{r['min']} | {r['max']} |")
    return md


def _find(d, sub, suffix):
    """The rocprofv3 output file ending in `suffix` under d/sub (it may sit in a
    per-host/per-process subdirectory)."""
    for root, _, files in os.walk(os.path.join(d, sub)):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    return None


HEADLINE_GRID = 256 * 512   # the 1.3B layer's forward: 256 workgroups of 8 waves


def summarize_profiles(d):
    """Write the profiles/ summaries from the rocprofv3 CSV outputs of PROFILE_COMMANDS
    run under directory d (each pass that is present)."""
    import csv
    import statistics

    def counters(sub, kernel, grid=None):
        """{counter name: [value per dispatch]} of the dispatches of `kernel` (and grid)."""
        path = _find(d, sub, "counter_collection.csv")
        out = {}
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"] and (grid is None or _grid(r) == grid):
                out.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return out

    from selective_state_space_79_amd.inputs import make_workload
    x = make_workload(3)
    head = "scan_fwd_kernel<unsigned short, 4, false, 0, true, 4, false, false>"
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    cmd = lambda k: PROFILE_COMMANDS[k].format(d=PROFILE_DIR)

    # kernel time, split by grid: the bench times several workloads with the same kernel
    stats_trace = _find(d, "stats", "kernel_trace.csv")
    if stats_trace:
        rows = _trace_rows(stats_trace)
        hr = [r for r in rows if head in r["name"] and r["grid"] == HEADLINE_GRID]
        md = ["# scan_fwd_kernel, mamba-1.3b-layer workload (4 x 4096 x 4096, N=16, bf16): rocprofv3 kernel times", "",
              f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
              "Command (from the repository root on the GPU box, after `cd /tmp && export TMPDIR=/tmp`):", "",
              "    " + cmd("stats"), "",
              "The default bench times several workloads; per-dispatch times from the kernel trace are grouped by "
              "kernel and grid size, so the headline forward (256 workgroups x 512 work-items = "
              f"{HEADLINE_GRID} work-items) has a row of its own.", ""]
        if hr:
            r = hr[0]
            md += [f"**Headline forward:** {r['calls']} dispatches, average {r['avg'] / 1e3:.1f} µs, median "
                   f"{r['median'] / 1e3:.1f} µs, min {r['min'] / 1e3:.1f} µs (warm-up dispatches included).", ""]
        md += _trace_table(rows)
        with open(os.path.join(ROOT, "profiles", "scan_fwd_mamba13b.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        ssd = [r for r in rows if "ssd_" in r["name"]]
        if ssd:
            src = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "ssd_fwd.hip")
            with open(src, "rb") as f:
                ssd_hash = hashlib.sha256(f.read()).hexdigest()[:16]
            scal = [r for r in rows if re.search(r"scan_fwd_kernel<[^,]+, \d+, true", r["name"])
                    or "scan_piece_states_kernel<128, false>" in r["name"] or "scan_carry_kernel" in r["name"]]
            md = ["# ssd_state_kernel + ssd_out_kernel, scalar-decay large-state workload with one step size per "
                  "head (batch 2, L 8192, 64 heads x 64, N 128, bf16): rocprofv3 kernel times", "",
                  f"Kernel source (`csrc/ssd_fwd.hip`) sha256[:16]: `{ssd_hash}`", "",
                  "From the same `--kernel-trace --stats` run of the default bench as `scan_fwd_mamba13b.md`; one "
                  "`ssm_ssd_fwd` call launches `ssd_gram_kernel`, `ssd_state_kernel` and `ssd_out_kernel`.  The "
                  "scalar-decay rows of the per-channel scan (same shapes) are listed below them.", "",
                  "Command (from the repository root on the GPU box):", "", "    " + cmd("stats"), ""]
            md += _trace_table(ssd + scal, 120)
            with open(os.path.join(ROOT, "profiles", "ssd_fwd_scalar_decay_head_dt.md"), "w") as f:
                f.write("\n".join(md) + "\n")

    # the chunked form of the scalar-decay scan (workload 5): kernel times from the stats
    # pass, occupancy and issue counters from their own pass
    chk_rows = [r for r in _trace_rows(stats_trace) if "scan_chunked_kernel" in r["name"]
                or ("scan_piece_states_kernel<128, false>" in r["name"]) or "scan_carry_kernel" in r["name"]] \
        if stats_trace else []
    ctr_path = _find(d, "chkctr", "counter_collection.csv")
    if chk_rows or ctr_path:
        x5 = make_workload(5)
        md = ["# Chunked form of the scalar-decay scan, per-channel step sizes (workload 5: batch 2, L 8192, dim "
              "4096 in 64 heads, N 128, bf16): rocprofv3 kernel times and counters", "",
              f"Kernel source (`csrc/scan_chunked.hip`) sha256[:16]: `{chunked_hash()}`", "",
              "One call launches `scan_piece_states_kernel<128, false>` (the end states of all pieces but the last, "
              "on the matrix cores), `scan_carry_kernel` (the pieces' starting states) and "
              "`scan_chunked_kernel<128>` (the full pass).", ""]
        if chk_rows:
            md += ["Kernel times, from the default bench's stats pass (all kernels of these names; the per-head "
                   "duality pass of `ssd_fwd_scalar_decay_head_dt.md` launches other kernels):", "",
                   "    " + cmd("stats"), ""]
            md += _trace_table(chk_rows, 100)
            md.append("")
        if ctr_path:
            c = {}
            for r in csv.DictReader(open(ctr_path)):
                c.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            md += ["Counters (medians per dispatch), command:", "", "    " + cmd("chunked_counters"), "",
                   "`GRBM_GUI_ACTIVE` is summed over the 8 XCDs (cycles = a eighth of it); `SQ_WAVE_CYCLES` counts "
                   "resident wave-cycles in units of 4 cycles; issue = 4 x (VALU + TRANS) SIMD-cycles over 1024 SIMDs.",
                   "", "| kernel | waves | cycles | waves/SIMD | VALU | TRANS | issue frac | MFMA busy | LDS instr |",
                   "|---|---|---|---|---|---|---|---|---|"]
            tot = {"SQ_INSTS_VALU": 0.0, "SQ_INSTS_VALU_TRANS_F32": 0.0}
            for name, cs in sorted(c.items(), key=lambda kv: -statistics.median(kv[1].get("SQ_INSTS_VALU", [0]))):
                med = {k: statistics.median(v) for k, v in cs.items()}
                cyc = med.get("GRBM_GUI_ACTIVE", 0) / 8
                if cyc <= 0:
                    continue
                for k in tot:
                    tot[k] += med.get(k, 0)
                iss = 4 * (med.get("SQ_INSTS_VALU", 0) + med.get("SQ_INSTS_VALU_TRANS_F32", 0)) / (SIMDS * cyc)
                md.append(f"| `{name[:90]}` | {med.get('SQ_WAVES', 0):.0f} | {cyc:.4g} | "
                          f"{4 * med.get('SQ_WAVE_CYCLES', 0) / (SIMDS * cyc):.2f} | {med.get('SQ_INSTS_VALU', 0):.4g} | "
                          f"{med.get('SQ_INSTS_VALU_TRANS_F32', 0):.4g} | {iss:.3f} | "
                          f"{med.get('SQ_VALU_MFMA_BUSY_CYCLES', 0) / (SIMDS * cyc):.3f} | {med.get('SQ_INSTS_LDS', 0):.4g} |")
            rec = {"kernels": sorted(c), "shape": [x5.batch, x5.L, x5.dim, x5.N],
                   "kernel_source_sha256_16": chunked_hash(), "command": cmd("chunked_counters"), **tot}
            with open(CHUNKED_FILE, "w") as f:
                json.dump(rec, f, indent=1)
        with open(os.path.join(ROOT, "profiles", "scan_chunked_scalar_decay.md"), "w") as f:
            f.write("\n".join(md) + "\n")

    # occupancy and matrix-core use of the duality pass's kernels
    if _find(d, "ssdctr", "counter_collection.csv"):
        src = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "ssd_fwd.hip")
        with open(src, "rb") as f:
            ssd_hash = hashlib.sha256(f.read()).hexdigest()[:16]
        md = ["# ssd_gram_kernel, ssd_state_(dma_)kernel, ssd_out_kernel: occupancy and matrix-core counters, scalar-decay "
              "large-state workload with one step size per head (batch 2, L 8192, 64 heads x 64, N 128, bf16)", "",
              f"Kernel source (`csrc/ssd_fwd.hip`) sha256[:16]: `{ssd_hash}`", "",
              "Command (from the repository root on the GPU box, after `cd /tmp && export TMPDIR=/tmp`):", "",
              "    " + cmd("ssd_counters"), "",
              "Medians per dispatch.  `GRBM_GUI_ACTIVE` is summed over the 8 XCDs, so the dispatch's cycles are a "
              "eighth of it; `SQ_WAVE_CYCLES` counts resident wave-cycles in units of 4 cycles; "
              "`SQ_VALU_MFMA_BUSY_CYCLES` sums the 1024 SIMDs' matrix-core busy cycles.  Derived: mean resident "
              "waves per SIMD = 4 x SQ_WAVE_CYCLES / (1024 x cycles); matrix-core busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles); LDS bank-conflict cycles per CU-cycle = "
              "SQ_LDS_BANK_CONFLICT / (256 x cycles).  Dispatch times under counter collection run longer than "
              "in `ssd_fwd_scalar_decay_head_dt.md`.", ""]
        names = [("ssd_gram_kernel", "C^T B per chunk"),
                 ("ssd_state_dma_kernel", "end states of the pieces, 16-byte rows straight to LDS"),
                 ("ssd_state_kernel", "end states of the pieces"), ("ssd_out_kernel", "outputs")]
        cols = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
        md += ["| kernel | " + " | ".join(cols) + " | cycles | waves/SIMD | MFMA busy | LDS conflict / CU-cycle |",
               "|---|" + "---|" * (len(cols) + 4)]
        for kname, what in names:
            c = counters("ssdctr", kname + "<128")
            if not c:
                continue
            med = {k: statistics.median(v) for k, v in c.items()}
            cyc = med.get("GRBM_GUI_ACTIVE", 0.0) / 8
            occ = 4 * med.get("SQ_WAVE_CYCLES", 0.0) / (1024 * cyc) if cyc else 0.0
            mfma = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * cyc) if cyc else 0.0
            lds = med.get("SQ_LDS_BANK_CONFLICT", 0.0) / (256 * cyc) if cyc else 0.0
            md.append(f"| `{kname}` ({what}) | " + " | ".join(f"{med.get(k, 0.0):.4g}" for k in cols) +
                      f" | {cyc:.4g} | {occ:.2f} | {mfma:.3f} | {lds:.3f} |")
        with open(os.path.join(ROOT, "profiles", "ssd_fwd_counters.md"), "w") as f:
            f.write("\n".join(md) + "\n")

    # instruction issue of the backward's role-split passes
    if _find(d, "bwdctr", "counter_collection.csv"):
        src = os.path.join(ROOT, "selective_state_space_79_amd", "csrc", "scan_bwd.hip")
        with open(src, "rb") as f:
            bwd_hash = hashlib.sha256(f.read()).hexdigest()[:16]
        md = ["# scan_bwd_ckpt_ws_kernel, scan_bwd_grad_ws_kernel: instruction-issue counters of the backward, "
              "mamba-1.3b-layer (4 x 4096 x 4096, N 16) and scalar-decay large-state (2 x 8192 x 4096, N 128) "
              "workloads, bf16", "",
              f"Kernel source (`csrc/scan_bwd.hip`) sha256[:16]: `{bwd_hash}`", "",
              "Command (from the repository root on the GPU box, after `cd /tmp && export TMPDIR=/tmp`):", "",
              "    " + cmd("bwd_counters"), "",
              "Medians per dispatch.  `GRBM_GUI_ACTIVE` is summed over the 8 XCDs, so the dispatch's cycles are an "
              "eighth of it.  A wave64 VALU instruction holds a SIMD16 for 4 cycles and a transcendental one for 8, "
              "so VALU issue = 4 x (SQ_INSTS_VALU + SQ_INSTS_VALU_TRANS_F32) / (1024 x cycles), the fraction of the "
              "1024 SIMDs' cycles spent issuing VALU work.  State updates per dispatch: 1.074e9 (N 16), 8.59e9 "
              "(N 128).", ""]
        cols = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32",
                "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"]
        md += ["| kernel | " + " | ".join(cols) + " | cycles | VALU issue | VALU per update |",
               "|---|" + "---|" * (len(cols) + 3)]
        shapes = [("scan_bwd_ckpt_ws_kernel<unsigned short, false, true, 4, 4, 16>", "checkpoints, N 16", 1.074e9),
                  ("scan_bwd_grad_ws_kernel<unsigned short, false, true, 4, 4, 16>", "gradients, N 16", 1.074e9),
                  ("scan_bwd_ckpt_ws_kernel<unsigned short, true, true, 16, 8, 8>", "checkpoints, N 128", 8.59e9),
                  ("scan_bwd_grad_ws_kernel<unsigned short, true, true, 16, 8, 8>", "gradients, N 128", 8.59e9)]
        for kname, what, upd in shapes:
            c = counters("bwdctr", kname)
            if not c:
                continue
            med = {k: statistics.median(v) for k, v in c.items()}
            cyc = med.get("GRBM_GUI_ACTIVE", 0.0) / 8
            issue = 4 * (med.get("SQ_INSTS_VALU", 0.0) + med.get("SQ_INSTS_VALU_TRANS_F32", 0.0)) / (1024 * cyc) if cyc else 0.0
            per = 64 * med.get("SQ_INSTS_VALU", 0.0) / upd
            md.append(f"| `{kname.split('<')[0]}` ({what}) | " + " | ".join(f"{med.get(k, 0.0):.4g}" for k in cols) +
                      f" | {cyc:.4g} | {issue:.3f} | {per:.1f} |")
        with open(os.path.join(ROOT, "profiles", "scan_bwd_counters.md"), "w") as f:
            f.write("\n".join(md) + "\n")

    # HBM traffic of the headline forward
    if _find(d, "fetch", "counter_collection.csv") and _find(d, "copyfetch", "counter_collection.csv"):
        alg = algorithmic_bytes(x)
        esz = 2
        alg_read = 3 * esz * x.batch * x.L * x.dim + 2 * esz * x.batch * x.N * x.L + 4 * (x.A.size + 2 * x.dim)
        alg_write = esz * x.batch * x.L * x.dim
        fetch = counters("fetch", head, HEADLINE_GRID)["FETCH_SIZE"]
        write = counters("write", head, HEADLINE_GRID)["WRITE_SIZE"]
        cfetch = [v for v in counters("copyfetch", "")["FETCH_SIZE"] if v > 1e5]
        cwrite = [v for v in counters("copywrite", "")["WRITE_SIZE"] if v > 1e5]
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
               "commands": [cmd(k) for k in ("fetch", "write", "copyfetch", "copywrite")]}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        md = ["# scan_fwd_kernel, mamba-1.3b-layer workload: HBM traffic per launch (rocprofv3 counters)", "",
              f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
              "`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, one run each; commands (repository root, GPU box):", ""]
        md += ["    " + c for c in rec["commands"]]
        md += ["", "Calibration: a plain 2 GiB device copy (`bench.py --calibrate-copy`) reads "
               f"{statistics.median(cfetch):.0f} KiB of FETCH_SIZE and {statistics.median(cwrite):.0f} KiB of "
               f"WRITE_SIZE per launch for {kib:.0f} KiB moved each way: scale factors {ffac:.4f} (fetch) and "
               f"{wfac:.4f} (write).", "",
               "| per launch | counter (KiB, median) | scaled bytes | algorithmic bytes | ratio |", "|---|---|---|---|---|",
               f"| read | {statistics.median(fetch):.0f} | {rd:.4g} | {alg_read:.4g} | {rd / alg_read:.3f} |",
               f"| write | {statistics.median(write):.0f} | {wr:.4g} | {alg_write:.4g} | {wr / alg_write:.3f} |",
               f"| total | | {rd + wr:.4g} | {alg:.4g} | {(rd + wr) / alg:.3f} |", ""]
        with open(os.path.join(ROOT, "profiles", "scan_fwd_mamba13b_traffic.md"), "w") as f:
            f.write("\n".join(md))
        print(json.dumps({"traffic_bytes_per_launch": rd + wr, "ratio_to_algorithmic": (rd + wr) / alg}))

    # VALU issue of the headline forward
    if _find(d, "valu", "counter_collection.csv"):
        c = counters("valu", head, HEADLINE_GRID)
        med = {k: statistics.median(v) for k, v in c.items()}
        trace = _find(d, "valu", "kernel_trace.csv")
        durs = [r for r in _trace_rows(trace) if head in r["name"] and r["grid"] == HEADLINE_GRID] if trace else []
        rec = {"kernel": head, "shape": [x.batch, x.L, x.dim, x.N], "kernel_source_sha256_16": kernel_hash(),
               "dispatches": len(c.get("SQ_INSTS_VALU", [])), "command": cmd("valu"), **med}
        with open(VALU_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        cyc = 4 * (med["SQ_INSTS_VALU"] + med["SQ_INSTS_VALU_TRANS_F32"])
        walk = 4 * 6 * x.updates / 64
        md = ["# VALU issue of the forward, mamba-1.3b-layer workload (4 x 4096 x 4096, N 16, bf16 I/O)", "",
              f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
              "Command (repository root on the GPU box, after `cd /tmp && export TMPDIR=/tmp`):", "",
              "    " + cmd("valu"), "",
              "Counters are totals per dispatch over all waves (median over the dispatches). A wave64 VALU "
              "instruction holds a SIMD16 for 4 cycles and a transcendental one (`SQ_INSTS_VALU_TRANS_F32`, also "
              "counted in `SQ_INSTS_VALU`) for 8, so the issue cycles are 4 x (VALU + TRANS), over 1024 SIMDs.", "",
              "| counter | per dispatch |", "|---|---|"]
        md += [f"| {k} | {v:.4g} |" for k, v in sorted(med.items())]
        md += ["", f"Issue cycles per call: {cyc:.4g}; the method's walk alone (6 slots per state update) needs "
               f"{walk:.4g}, so the kernel issues {cyc / walk:.3f}x its walk floor.",
               f"At 2.4 GHz over 1024 SIMDs that is {cyc / (SIMDS * CLOCK_HZ) * 1e6:.1f} µs of issue per call."]
        if durs:
            md.append(f"Dispatch time in this (profiled) run: median {durs[0]['median'] / 1e3:.1f} µs.")
        # every kernel of the run (the forward, and the backward's passes, timed in the same run)
        allc = {}
        for r in csv.DictReader(open(_find(d, "valu", "counter_collection.csv"))):
            allc.setdefault((r["Kernel_Name"], _grid(r)), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        md += ["", "All kernels of the run (medians per dispatch; issue = 4 x (VALU + TRANS) cycles at 2.4 GHz over "
               "1024 SIMDs):", "", "| kernel | grid | dispatches | SQ_INSTS_VALU | TRANS_F32 | SQ_INSTS_LDS | issue µs |",
               "|---|---|---|---|---|---|---|"]
        for (name, grid), cs in sorted(allc.items(), key=lambda kv: -statistics.median(kv[1].get("SQ_INSTS_VALU", [0]))):
            v = statistics.median(cs.get("SQ_INSTS_VALU", [0]))
            t = statistics.median(cs.get("SQ_INSTS_VALU_TRANS_F32", [0]))
            if v < 1e6:
                continue
            md.append(f"| `{name[:100]}` | {grid} | {len(cs.get('SQ_INSTS_VALU', []))} | {v:.4g} | {t:.4g} | "
                      f"{statistics.median(cs.get('SQ_INSTS_LDS', [0])):.4g} | {4 * (v + t) / (SIMDS * CLOCK_HZ) * 1e6:.1f} |")
        with open(os.path.join(ROOT, "profiles", "scan_fwd_mamba13b_valu_issue.md"), "w") as f:
            f.write("\n".join(md) + "\n")

    conv_trace = _find(d, "convstats", "kernel_trace.csv")
    if conv_trace:
        md = ["# Fused convolution front end + scan, mamba-1.3b-layer workload (4 x 4096 x 4096, N=16, bf16, "
              "width-4 SiLU convolution): rocprofv3 kernel times", "",
              f"Kernel source sha256[:16]: `{kernel_hash()}`", "",
              "The run times the plain scan first and then the fused front end (`ssm_selective_scan_fwd_conv`, "
              "then the fused decode step); the fused scan is its own instantiation (template flag).", "",
              "Command (from the repository root on the GPU box):", "", "    " + cmd("conv_stats"), ""]
        md += _trace_table(_trace_rows(conv_trace))
        with open(os.path.join(ROOT, "profiles", "scan_fwd_conv_mamba13b.md"), "w") as f:
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

    def call(i):
        st = fn(*args)
        if st != 0:
            raise ssm.SsmError(st, "ssm_selective_scan_step")

    t = time_calls(call, steps, warmup, stream)
    us = t["ms_events"] * 1e3
    # algorithmic bytes: state read + written, A once, u/delta/z read and y written,
    # B and C per sequence, D and dt_bias once
    nbytes = 8 * batch * dim * N + 4 * dim * N + 8 * batch * dim + 4 * batch * N + 8 * dim
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"mamba-1.3b-layer decode step, {batch} sequences (dim {dim}, N {N}, bf16 I/O, fp32 state)",
            "us_per_step": round(us, 3), "tokens_per_s": round(batch / (us * 1e-6), 1),
            "updates_per_s": batch * dim * N / (us * 1e-6), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm",
            "us_median": round(t["ms_median"] * 1e3, 3), "us_min": round(t["ms_min"] * 1e3, 3)}


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
        def c(i):
            st = call()
            if st != 0:
                raise ssm.SsmError(st, "fused conv")
        return time_calls(c, n, nw, stream)["ms_events"]

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
# with a scalar decay per head the decay is one exp2 per (b,t,d), shared by the state
# entries: the recompute (x*B mul, state fma, read-out fma for the gate's derivative),
# the reverse step (g fma, e = a*g mul, sums of g*a*h_prev and g*B: 2 fma; ds*h and g*x
# for dC, dB: 2 mul) and the channel sums of dB, dC (2 add)
BWD_OPS_PER_UPDATE_SCALAR = 11


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

    def call(i):
        st = fn(*args)
        if st != 0:
            raise ssm.SsmError(st, "ssm_selective_scan_bwd")

    tb = time_calls(call, steps, warmup, stream)
    ms = tb["ms_events"]
    esz = 2 if x.io == "bf16" else 4
    # u, delta, z, dy read and du, ddelta, dz written per element; B, C read and dB, dC
    # (float32) written per (b, t, n); A, D, dt_bias read and dA, dD, ddt_bias written
    nbytes = (7 * esz * x.batch * x.L * x.dim + (2 * esz + 8) * x.batch * x.N * x.L
              + 8 * (x.A.size + 2 * x.dim))
    ops = BWD_OPS_PER_UPDATE_SCALAR if x.nheads else BWD_OPS_PER_UPDATE
    tops = ops * x.updates / (ms * 1e-3) / 1e12
    rec = {"workload": f"{x.batch}x{x.L}x{x.dim}, N {x.N}, {x.io} I/O" + (f", {x.nheads} heads scalar decay" if x.nheads else "")
                       + ": gradients of every input",
           "ms_per_call": round(ms, 4), "updates_per_s": x.updates / (ms * 1e-3), "plan": plan,
           "roofline": {"bound": "alu", "achieved": round(tops, 3), "peak": round(VALU_PEAK_TOPS, 2),
                        "unit": "TFLOP/s", "frac": round(tops / VALU_PEAK_TOPS, 4),
                        "note": f"{ops} fp32 VALU lane operations per state update"},
           "algorithmic_bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "ms_median": round(tb["ms_median"], 4), "ms_min": round(tb["ms_min"], 4)}

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
            def c(i):
                st = fn(*a)
                if st != 0:
                    raise ssm.SsmError(st, name)
            return time_calls(c, steps, warmup, stream)["ms_events"]

        f_ms = timed(lib.ssm_selective_scan_fwd_ckpt, fargs, "ssm_selective_scan_fwd_ckpt")
        b_ms = timed(lib.ssm_selective_scan_bwd_ckpt, bargs, "ssm_selective_scan_bwd_ckpt")
        rec["with_forward_checkpoints"] = {
            "fwd_ckpt_ms": round(f_ms, 4), "bwd_ckpt_ms": round(b_ms, 4), "checkpoint_bytes": nck,
            "note": "ssm_selective_scan_fwd_ckpt keeps the state every 16 steps; ssm_selective_scan_bwd_ckpt "
                    "starts from them and skips its own recomputation walk"}
    return rec




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

    def timed(call, n, w, full=False):
        def c(i):
            st = call()
            if st != 0:
                raise ssm.SsmError(st, "bench call")
        t = time_calls(c, n, w, stream)
        return t if full else t["ms_events"]

    tss = timed(lambda: fn(*args), steps, warmup, full=True)
    ms = tss["ms_events"]
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
            "ms_per_call": round(ms, 4), "ms_median": round(tss["ms_median"], 4), "ms_min": round(tss["ms_min"], 4),
            "updates_per_s": x.updates / (ms * 1e-3), "plan": plan,
            "hbm": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_call": nbytes},
            "mfma": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "note": "bf16 matrix FLOPs the chunked method issues (operands split in two bf16 parts)"},
            "per_channel_scan_same_inputs": {"ms_per_call": round(ms_scan, 4),
                                             "updates_per_s": x.updates / (ms_scan * 1e-3),
                                             "speedup_of_chunked": round(ms_scan / ms, 2)}}


def progress(msg: str):
    """One line on stderr per finished stage (the JSON line on stdout stays alone)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    global MIN_WARMUP_S
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
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other named workloads (tiny, 130M layer, long sequence, scalar decay N=128)")
    ap.add_argument("--no-linear", action="store_true", help="skip the linear-in-L check")
    ap.add_argument("--only-workloads", default="", help="comma-separated indices of the other workloads to time "
                    "(default: all but the headline)")
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S,
                    help="least wall time of untimed warm-up before each timed loop (seconds)")
    ap.add_argument("--calibrate-copy", action="store_true", help="only run a 2 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR", help="write profiles/ summaries from rocprofv3 CSVs in DIR")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    MIN_WARMUP_S = args.min_warmup_s

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
    rec_main = scan_workload_bench(x, dev, args.steps, args.warmup, stream)
    progress(f"workload {args.workload} timed: {rec_main['timing']['ms_per_step']:.4f} ms per call")
    t = rec_main["timing"]
    ms_per_step = t["ms_per_step"]
    updates = x.updates
    value = updates / (ms_per_step * 1e-3)
    plan = rec_main["plan"]
    traffic = measured_traffic() if (args.workload == 3 and plan["nchunks"] == 1) else None
    rec_main["roofline"]["traffic"] = traffic
    rec_main["hbm"]["traffic"] = traffic
    t.update({"input_gen_s": round(gen_s, 2), "kernel_source_sha256_16": kernel_hash(),
              "device": torch.cuda.get_device_name(0)})

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
        "hbm_gbs": rec_main["hbm"]["achieved"],
        "hbm_frac": rec_main["hbm"]["frac"],
        "roofline": rec_main["roofline"],
        "hbm": rec_main["hbm"],
        "timing": t,
    }
    if rec_main.get("valu_issue"):
        rec["valu_issue"] = rec_main["valu_issue"]
    if args.workload == 3 and not args.no_decode:
        rec["decode_step"] = [decode_step_bench(64), decode_step_bench(256)]
        progress("decode step timed")
    if args.fused_conv:
        rec["fused_conv"] = fused_conv_bench(x, dev)
    if not args.no_backward:
        rec["backward"] = backward_bench(x, dev)
        progress("backward timed")
        if args.workload != 5:
            # the scalar-decay N = 128 shapes (workload 5, per-channel step sizes)
            from selective_state_space_79_amd.inputs import make_workload as _mw
            x5 = _mw(5)
            d5 = to_device(x5, "cuda:0")
            rec["backward_scalar_decay_n128"] = backward_bench(x5, d5, steps=10, warmup=3)
            progress("scalar-decay backward timed")
            del d5, x5
            torch.cuda.empty_cache()
    if not args.no_ssd:
        del dev
        torch.cuda.empty_cache()
        rec["ssd"] = ssd_bench()
        progress("duality pass timed")
    if not args.no_linear:
        rec["linear_in_L"] = linear_in_L_bench(args.steps, args.warmup, stream)
        progress("linear-in-L timed")
    if not args.no_workloads:
        others = [i for i in (1, 2, 3, 4, 5) if i != args.workload]
        if args.only_workloads:
            others = [i for i in others if str(i) in args.only_workloads.split(",")]
        rec["workloads"] = other_workloads_bench(others, args.steps, args.warmup, stream)
        progress("other workloads timed")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_batches)
        progress("cpu baseline timed")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
