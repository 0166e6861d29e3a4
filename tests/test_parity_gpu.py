"""GPU parity: the HIP scan (through the C ABI) against the fp64 oracle.

Inputs are seeded and synthetic (selective_state_space_79_amd.inputs).  Small and
ragged shapes, and the five named workloads at full size in the launch
configuration the benchmark uses, are compared element by element over the whole
output (at full size the oracle runs block by block of channels).
"""
import math
import sys

import numpy as np
import pytest

from scan_cases import TOL, oracle_err_all, rel_err, run_gpu, run_oracle
from selective_state_space_79_amd.inputs import ScanInputs, make_inputs, make_workload

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def test_worked_example_through_abi():
    """The qubittool scalar example (retain/write/read) as a one-state scan:
    A = -1, dt = -ln(retain) via its inverse softplus, B = write/dt, u = value, C = 1."""
    announce("worked example f32 (1,3,1,1)")
    value = np.array([2.0, 9.0, 1.0])
    retain = np.array([0.10, 0.95, 0.50])
    write = np.array([1.0, 0.0, 1.0])
    dt = -np.log(retain)
    delta = np.array([math.log(math.expm1(v)) for v in dt])
    f = lambda a: np.asarray(a, dtype=np.float32).reshape(1, 1, 3)
    x = ScanInputs(1, 3, 1, 1, 0, "f32", f(value), f(delta), f(np.zeros(3)), f(write / dt), f(np.ones(3)),
                   np.array([[-1.0]], dtype=np.float32), np.zeros(1, np.float32), np.zeros(1, np.float32))
    y = run_gpu(x, with_D=False, with_z=False, with_bias=False)
    np.testing.assert_allclose(y.reshape(-1), [2.0, 1.9, 1.95], rtol=0, atol=2e-6)
    yref = run_oracle(x, with_D=False, with_z=False, with_bias=False)
    assert rel_err(y, yref) < 2e-6


def test_tiny_fp32_workload():
    x = make_workload(1)
    announce(f"workload 1 {x.batch, x.L, x.dim, x.N} f32")
    y = run_gpu(x)
    err = rel_err(y, run_oracle(x))
    print(f"workload 1 err={err:.3e}", flush=True)
    assert err <= TOL["f32"]


# (batch, L, dim, N, io, nheads, with_D, with_z, with_bias, nchunks, states_per_lane)
RAGGED = [
    (1, 1, 1, 1, "f32", 0, True, True, True, 0, 0),
    (1, 7, 3, 2, "f32", 0, True, True, True, 0, 0),
    (2, 33, 65, 4, "f32", 0, True, True, True, 0, 0),
    (1, 100, 64, 16, "f32", 0, True, False, True, 0, 0),
    (3, 257, 130, 16, "bf16", 0, True, True, True, 0, 0),
    (2, 64, 63, 16, "bf16", 0, False, True, False, 0, 0),
    (1, 200, 129, 3, "bf16", 0, True, True, True, 0, 0),
    (1, 96, 64, 5, "f32", 0, True, True, True, 0, 0),
    (2, 128, 72, 16, "bf16", 4, True, True, True, 0, 0),
    (1, 160, 128, 128, "bf16", 8, True, True, True, 0, 0),
    (1, 48, 64, 128, "bf16", 0, True, True, True, 0, 0),
    (1, 40, 64, 256, "bf16", 0, True, True, True, 0, 0),
    (1, 40, 70, 256, "f32", 2, True, True, True, 0, 0),
    # pieces along L: every carry path, ragged last piece
    (1, 1000, 64, 16, "bf16", 0, True, True, True, 2, 0),
    (2, 777, 100, 16, "f32", 0, True, True, True, 5, 0),
    (1, 999, 64, 4, "bf16", 0, True, True, True, 31, 0),
    (1, 512, 64, 128, "bf16", 4, True, True, True, 3, 0),
    # scalar decay, bf16, pieces: the pieces' end states on the matrix cores (32 and 64
    # states; channels beyond dim in the last block; pieces not whole 64-step chunks)
    (2, 1024, 64, 32, "bf16", 2, True, True, True, 5, 0),
    (1, 640, 96, 64, "bf16", 3, False, True, True, 4, 0),
    (1, 300, 65, 16, "f32", 0, True, True, True, 7, 0),
    # forced states per lane
    (1, 80, 64, 16, "bf16", 0, True, True, True, 0, 1),
    (1, 80, 64, 16, "bf16", 0, True, True, True, 0, 2),
    (1, 80, 64, 16, "f32", 0, True, True, True, 0, 8),
    (1, 80, 64, 16, "f32", 0, True, True, True, 0, 16),
    (1, 80, 64, 24, "bf16", 0, True, True, True, 0, 16),
    (1, 80, 64, 64, "bf16", 0, True, True, True, 3, 4),
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "b{}L{}d{}N{}{}h{}D{}z{}bias{}ch{}spl{}".format(*[int(v) if isinstance(v, bool) else v for v in c]))
def test_ragged_shapes(case):
    batch, L, dim, N, io, nheads, wD, wz, wb, nch, spl = case
    seed = 1000 + RAGGED.index(case)
    announce(f"ragged {case} seed={seed}")
    x = make_inputs(batch, L, dim, N, seed=seed, io=io, nheads=nheads)
    y = run_gpu(x, with_D=wD, with_z=wz, with_bias=wb, nchunks=nch, states_per_lane=spl)
    yref = run_oracle(x, with_D=wD, with_z=wz, with_bias=wb)
    err = rel_err(y, yref)
    print(f"err={err:.3e}", flush=True)
    assert np.all(np.isfinite(y))
    assert err <= TOL[io]


@pytest.mark.parametrize("index", [2, 3, 4, 5])
def test_full_size_workload_all_outputs(index):
    """Full-size run in the benchmark's launch configuration (library-chosen plan),
    every output element compared with the oracle (computed block by block of
    channels)."""
    import selective_state_space_79_amd as ssm

    x = make_workload(index)
    plan = ssm.ssm_selective_scan_plan(ssm.make_dims(x.batch, x.L, x.dim, x.N, nheads=x.nheads)).as_dict()
    announce(f"workload {index} {(x.batch, x.L, x.dim, x.N, x.nheads)} full size, plan {plan['nchunks']} pieces")
    y = run_gpu(x)
    assert np.all(np.isfinite(y))
    err, count = oracle_err_all(x, y)
    print(f"workload {index} all {count} outputs: max err={err:.3e} (bar {TOL[x.io]:g})", flush=True)
    assert count == x.batch * x.dim * x.L
    assert err <= TOL[x.io]


@pytest.mark.parametrize("shape", [(3, 8192, 1024, 16), (2, 16384, 2560, 16)])
def test_round_filling_piece_counts_all_outputs(shape):
    """Shapes whose library-chosen piece count fills whole rounds of workgroups (48 and
    80 channel blocks: 16 and 9 pieces), every output checked."""
    import selective_state_space_79_amd as ssm

    x = make_inputs(*shape, seed=sum(shape), io="bf16")
    plan = ssm.ssm_selective_scan_plan(ssm.make_dims(*shape)).as_dict()
    announce(f"round-filling pieces {shape} plan {plan['nchunks']} pieces")
    assert plan["nchunks"] in (16, 9)
    y = run_gpu(x)
    err, count = oracle_err_all(x, y)
    print(f"{shape} all {count} outputs: err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_extreme_values(io):
    """Step sizes from ~1e-35 to ~80 (fully decayed steps, denormal step sizes),
    saturated gates (|z| up to 60), zero decay on some entries and zero input on
    some steps."""
    announce(f"extreme values (2, 300, 70, 16) {io}")
    x = make_inputs(2, 300, 70, 16, seed=2024, io=io)
    rng = np.random.default_rng(5)
    scale = rng.choice([1.0, 8.0, 25.0, 60.0], size=x.delta.shape).astype(np.float32)
    x.delta = (x.delta * scale).astype(np.float32)
    x.delta[:, :, 10] = 80.0
    x.delta[:, :, 11] = -80.0
    x.z = (x.z * rng.choice([1.0, 30.0, 60.0], size=x.z.shape)).astype(np.float32)
    x.A[:, 3] = 0.0
    x.B[:, :, 50:60] = 0.0
    if io == "bf16":
        from selective_state_space_79_amd.inputs import round_to_bf16
        x.delta, x.z = round_to_bf16(x.delta), round_to_bf16(x.z)
    # Here the states grow to ~1.4e3 and largely cancel in the read-out, so with fp32
    # state the absolute error of O(1) outputs is set by eps32 * N * |C.h| ~ 1e-3: a
    # plain fp32 evaluation of the recurrence (numpy) misses 1e-4 by the same margin
    # (5.9e-4).  The f32 bar for these inputs is therefore 1e-3; bf16 keeps 2e-2.
    tol = 1e-3 if io == "f32" else TOL[io]
    for nch in (0, 3):
        y = run_gpu(x, nchunks=nch)
        yref = run_oracle(x)
        err = rel_err(y, yref)
        print(f"nchunks={nch} err={err:.3e}", flush=True)
        assert np.all(np.isfinite(y))
        assert err <= tol


def test_maximum_piece_count():
    """SSM_MAX_CHUNKS (1024) forced on a 32768-step sequence: 1024 one-tile pieces,
    1023 carries composed in sequence."""
    announce("1024 pieces (1, 32768, 64, 16) bf16")
    x = make_inputs(1, 32768, 64, 16, seed=31, io="bf16", dt_range=(1e-4, 1e-2))
    import selective_state_space_79_amd as ssm

    dims = ssm.make_dims(1, 32768, 64, 16, nchunks=1024)
    assert ssm.ssm_selective_scan_plan(dims).nchunks == 1024
    y = run_gpu(x, nchunks=1024)
    err, count = oracle_err_all(x, y)
    print(f"all {count} outputs: err={err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("N,spl,nheads", [(5, 2, 0), (33, 4, 0), (100, 16, 0), (48, 0, 3), (7, 0, 7)])
def test_padded_state_counts(N, spl, nheads):
    """dstate values that do not fill the workgroup's waves (padding entries)."""
    announce(f"padded states N={N} spl={spl} nheads={nheads}")
    x = make_inputs(1, 96, 21 * max(nheads, 1), N, seed=100 + N, io="f32", nheads=nheads)
    y = run_gpu(x, states_per_lane=spl)
    err = rel_err(y, run_oracle(x))
    print(f"err={err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_library_loaded_before_torch():
    """A process whose first call into the library (a plan query) comes before torch is
    imported still runs the scan: the binding loads torch's HIP runtime first, so the
    library and torch share one runtime."""
    import subprocess

    code = ("import sys; sys.path.insert(0, {root!r})\n"
            "import selective_state_space_79_amd as ssm\n"
            "ssm.ssm_selective_scan_plan(ssm.make_dims(3, 8192, 1024, 16))\n"
            "from selective_state_space_79_amd.inputs import make_inputs, to_device\n"
            "import torch\n"
            "x = make_inputs(3, 8192, 1024, 16, seed=5, io='bf16'); d = to_device(x)\n"
            "y = ssm.selective_scan_fwd(d['u'], d['delta'], d['A'], d['B'], d['C'], d['D'], d['z'], d['dt_bias'])\n"
            "torch.cuda.synchronize(); print('scan ok', bool(torch.isfinite(y.float()).all()))\n")
    root = __file__.rsplit("/tests/", 1)[0]
    announce("library loaded before torch, in a child process")
    r = subprocess.run([sys.executable, "-c", code.format(root=root)], capture_output=True, text=True, timeout=300)
    print(r.stdout[-500:], r.stderr[-500:], flush=True)
    assert r.returncode == 0 and "scan ok True" in r.stdout
