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
