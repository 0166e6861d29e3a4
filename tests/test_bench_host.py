"""Host-side checks of bench.py's bookkeeping (no GPU): the one-GPU refusal, the
algorithmic byte count of the 1.3B-layer workload, and that measured HBM traffic is
reported only for the kernel source it was taken on."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_mamba_1_3b_layer():
    # u, delta, z read and y written in bf16 per (b, t, d); B and C in bf16 per
    # (b, t, n); A (dim x N), D and dt_bias in fp32 once.
    x = SimpleNamespace(io="bf16", batch=4, L=4096, dim=4096, N=16, A=np.zeros((4096, 16), np.float32))
    expected = 4 * 2 * 4 * 4096 * 4096 + 2 * 2 * 4 * 16 * 4096 + 4 * (4096 * 16 + 2 * 4096)
    assert bench.algorithmic_bytes(x) == expected == 538_214_400
    x32 = SimpleNamespace(io="f32", batch=1, L=64, dim=4, N=4, A=np.zeros((4, 4), np.float32))
    assert bench.algorithmic_bytes(x32) == 4 * 4 * 64 * 4 + 2 * 4 * 4 * 64 + 4 * (16 + 8)


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic() is None  # no file
    path.write_text("not json")
    assert bench.measured_traffic() is None
    path.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_hash(), "hbm_bytes_per_launch": 5.5e8}))
    assert bench.measured_traffic() == 5.5e8
    other = "0" * 16 if bench.kernel_hash() != "0" * 16 else "1" * 16
    path.write_text(json.dumps({"kernel_source_sha256_16": other, "hbm_bytes_per_launch": 5.5e8}))
    assert bench.measured_traffic() is None


def test_kernel_trace_rows_split_by_grid(tmp_path):
    """The profile summary groups dispatches by kernel and grid size, so the headline
    forward's row is not mixed with another workload's calls of the same kernel."""
    path = tmp_path / "scan_kernel_trace.csv"
    rows = ["Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp"]
    for i in range(3):
        rows.append(f"k<a>,{bench.HEADLINE_GRID},1,1,{1000 * i},{1000 * i + 300}")
    rows.append("k<a>,98304,1,1,5000,5150")
    path.write_text("\n".join(rows) + "\n")
    got = {(r["name"], r["grid"]): r for r in bench._trace_rows(str(path))}
    head = got[("k<a>", bench.HEADLINE_GRID)]
    assert head["calls"] == 3 and head["avg"] == 300 and head["min"] == 300
    assert got[("k<a>", 98304)]["calls"] == 1 and got[("k<a>", 98304)]["avg"] == 150


def test_valu_issue_needs_the_profiled_source_and_shape(tmp_path, monkeypatch):
    path = tmp_path / "valu.json"
    monkeypatch.setattr(bench, "VALU_FILE", str(path))
    x = SimpleNamespace(batch=4, L=4096, dim=4096, N=16, updates=4 * 4096 * 4096 * 16)
    assert bench.measured_valu_issue(x, 0.3) is None
    rec = {"kernel_source_sha256_16": bench.kernel_hash(), "shape": [4, 4096, 4096, 16],
           "SQ_INSTS_VALU": 1.2e8, "SQ_INSTS_VALU_TRANS_F32": 2.1e7}
    path.write_text(json.dumps(rec))
    vi = bench.measured_valu_issue(x, 0.3)
    assert abs(vi["issue_frac"] - 4 * 1.41e8 / (1024 * 2.4e9 * 0.3e-3)) < 1e-3
    # the walk floor: 6 issue slots per state update, wave64 instructions of 4 cycles
    assert abs(vi["walk_floor_issue_frac"] - 4 * 6 * x.updates / 64 / (1024 * 2.4e9 * 0.3e-3)) < 1e-3
    rec["shape"] = [8, 2048, 1536, 16]
    path.write_text(json.dumps(rec))
    assert bench.measured_valu_issue(x, 0.3) is None


def test_chunked_form_counts(tmp_path, monkeypatch):
    """Matrix work of the chunked form on the scalar-decay N = 128 workload (128 channel
    blocks x 512 chunks of 16 steps; pieces of 1376 steps, the aggregate over five), and
    its VALU issue reported only for the profiled source and shape."""
    x = SimpleNamespace(batch=2, L=8192, dim=4096, N=128)
    plan = {"nchunks": 6, "chunk_len": 1376}
    gram = 2 * 16 * 16 * 128                 # C^T B, in each of the 4 waves
    read = 2 * 16 * 64 * 128                 # state read, one part
    update = 2 * 128 * 64 * 16               # state update, one part
    agg = 2 * 128 * 64                       # aggregate, per step and part
    assert bench.chunked_mfma_flops(x, plan) == 128 * 512 * (4 * gram + 2 * read + 2 * update) + 128 * 5 * 1376 * 2 * agg
    path = tmp_path / "chk.json"
    monkeypatch.setattr(bench, "CHUNKED_FILE", str(path))
    assert bench.measured_chunked_issue(x, 0.4) is None
    rec = {"kernel_source_sha256_16": bench.chunked_hash(), "shape": [2, 8192, 4096, 128],
           "SQ_INSTS_VALU": 1.3e8, "SQ_INSTS_VALU_TRANS_F32": 8e6}
    path.write_text(json.dumps(rec))
    vi = bench.measured_chunked_issue(x, 0.4)
    assert abs(vi["issue_frac"] - 4 * 1.38e8 / (1024 * 2.4e9 * 0.4e-3)) < 1e-3
    rec["kernel_source_sha256_16"] = "0" * 16 if bench.chunked_hash() != "0" * 16 else "1" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_chunked_issue(x, 0.4) is None
