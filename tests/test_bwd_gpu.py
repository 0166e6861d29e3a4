"""GPU parity of the backward pass (ssm_selective_scan_bwd) against the oracle's fp64
gradients (oracle.selective_scan_bwd), on seeded synthetic inputs and cotangents.

Tolerances.  With float32 I/O every gradient must be within 1e-4 (the forward's bar).
With bf16 I/O, du, ddelta and dz are rounded to bf16 (relative error up to 2^-9), so
they get the forward's bf16 bar of 2e-2; the float32 outputs (dA, dB, dC, dD,
ddt_bias, dh0) are computed in float32 from inputs the oracle sees exactly, so they
keep 1e-4.  Per-element outputs use |g - r| / max(1, |r|); sums over many terms use
the error relative to the tensor's largest magnitude (see bwd_cases.py).
"""
import sys

import numpy as np
import pytest

from bwd_cases import ELEMENTWISE, compare, run_gpu_bwd, run_oracle_bwd
from selective_state_space_79_amd.inputs import ScanInputs, make_cotangents, make_inputs, make_workload

pytestmark = pytest.mark.gpu

F32_OUT_TOL = 1e-4


def announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_for(io, name):
    if io == "bf16" and name in ("du", "ddelta", "dz"):
        return 2e-2
    return 1e-4


def check(x, g, r, label=""):
    errs = compare(g, r)
    print(label + " " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in g.items():
        assert np.all(np.isfinite(v)), k
    for k, e in errs.items():
        assert e <= tol_for(x.io, k), (k, e)
    return errs


# (batch, L, dim, N, io, nheads, with_opts, h0, dh_last, nchunks, states_per_lane)
CASES = [
    (1, 1, 1, 1, "f32", 0, True, True, True, 0, 0),
    (1, 64, 4, 4, "f32", 0, True, True, True, 0, 0),
    (1, 64, 4, 4, "f32", 0, False, False, False, 0, 0),
    (2, 100, 70, 16, "f32", 0, True, False, False, 0, 0),
    (2, 257, 130, 16, "bf16", 0, True, False, False, 0, 0),
    (3, 33, 65, 3, "f32", 0, True, True, False, 0, 0),
    (1, 96, 64, 5, "f32", 0, False, False, True, 0, 0),
    (1, 150, 64, 40, "f32", 0, True, False, False, 0, 0),
    (1, 100, 64, 100, "f32", 0, True, False, False, 0, 0),
    (1, 90, 70, 128, "f32", 0, True, True, True, 0, 0),
    (1, 200, 96, 128, "bf16", 4, True, True, False, 0, 0),
    (2, 128, 72, 16, "bf16", 4, True, False, True, 0, 0),
    (1, 160, 126, 7, "f32", 7, True, True, True, 0, 0),
    # 9..16 entries: padded to 16 in the gradient pass with helper waves
    (1, 203, 100, 12, "bf16", 0, True, True, True, 0, 0),
    (1, 130, 64, 9, "f32", 2, True, False, True, 2, 0),
    # pieces along L (forward and reverse carries), ragged last piece
    (1, 300, 64, 16, "f32", 0, False, True, True, 4, 0),
    (2, 1000, 64, 16, "bf16", 0, False, True, True, 5, 0),
    (1, 999, 65, 4, "bf16", 0, True, False, False, 31, 0),
    (1, 512, 64, 128, "bf16", 8, True, True, True, 3, 0),
    # scalar decay, bf16, pieces: the pieces' aggregates on the matrix cores (32 and 64
    # states; without the gate; channels beyond dim in the last block)
    (2, 1024, 64, 32, "bf16", 2, True, True, True, 5, 0),
    (1, 640, 96, 64, "bf16", 3, False, False, True, 4, 0),
    # 65..128 entries with scalar decay: role-split gradient pass, entries in groups of 4
    # (padding entries inside the last groups with N = 100; float32 rows)
    (1, 136, 64, 100, "f32", 2, True, True, True, 0, 0),
    (2, 264, 130, 128, "bf16", 2, True, True, True, 0, 0),
    # forced states per lane
    (1, 80, 64, 4, "f32", 0, True, False, False, 0, 1),
    (1, 80, 64, 16, "f32", 0, True, False, False, 0, 4),
    (1, 80, 64, 40, "f32", 0, True, False, False, 0, 8),
    (1, 80, 64, 100, "f32", 0, True, False, False, 0, 16),
    (1, 77, 64, 24, "bf16", 0, True, True, True, 0, 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}L{}d{}N{}{}h{}o{}h0{}dh{}ch{}spl{}".format(
    *[int(v) if isinstance(v, bool) else v for v in c]))
def test_backward_matches_oracle(case):
    batch, L, dim, N, io, nheads, opts, with_h0, with_dhl, nch, spl = case
    seed = 2000 + CASES.index(case)
    announce(f"bwd {case} seed={seed}")
    x = make_inputs(batch, L, dim, N, seed=seed, io=io, nheads=nheads)
    dy, dhl = make_cotangents(x, seed=seed + 1, with_dh_last=with_dhl)
    h0 = np.random.default_rng(seed + 2).standard_normal((batch, dim, N)).astype(np.float32) if with_h0 else None
    kw = dict(with_D=opts, with_z=opts, with_bias=opts)
    g = run_gpu_bwd(x, dy, h0=h0, dh_last=dhl, nchunks=nch, states_per_lane=spl, **kw)
    r = run_oracle_bwd(x, dy, h0=h0, dh_last=dhl, **kw)
    check(x, g, r)
    if not opts:
        assert "dz" not in g


@pytest.mark.parametrize("index", [1, 2, 3])
def test_backward_full_size_workloads(index):
    """Workloads 1-3 at full size in the library-chosen plan, every gradient against
    the oracle's (all rows)."""
    x = make_workload(index)
    announce(f"bwd workload {index} {(x.batch, x.L, x.dim, x.N)} full")
    dy, _ = make_cotangents(x, seed=50 + index)
    g = run_gpu_bwd(x, dy)
    r = run_oracle_bwd(x, dy)
    check(x, g, r, f"workload {index}")


def _as_f32(x: ScanInputs) -> ScanInputs:
    return ScanInputs(x.batch, x.L, x.dim, x.N, x.nheads, "f32", x.u, x.delta, x.z, x.B, x.C, x.A, x.D, x.dt_bias)


@pytest.mark.parametrize("index", [4, 5])
def test_backward_full_size_sampled_and_identities(index):
    """Workloads 4 and 5 at full size: the per-channel gradients of sampled channels
    against the oracle on those channels, and dB, dC, du against the homogeneity
    identities  sum dy*y = <dC,C> + <dD,D> = <dB,B> + <dD,D> = <du,u>  (zero start,
    no final-state gradient), with y from the float32 forward on the same values."""
    import torch
    from scan_cases import run_gpu

    x = make_workload(index)
    announce(f"bwd workload {index} {(x.batch, x.L, x.dim, x.N, x.nheads)} full")
    dy, _ = make_cotangents(x, seed=50 + index)
    g = run_gpu_bwd(x, dy)
    for k, v in g.items():
        assert np.all(np.isfinite(v)), k
    rng = np.random.default_rng(index)
    hd = x.dim // x.nheads if x.nheads else 1
    if x.nheads:
        chans = np.sort(np.concatenate([np.arange(hd), x.dim - hd + np.arange(hd)]))   # two whole heads
    else:
        chans = np.unique(np.concatenate([[0, x.dim - 1], rng.integers(0, x.dim, 10)]))
    r = run_oracle_bwd(x, dy, channels=chans)
    sub = {k: g[k][:, chans] for k in ("du", "ddelta", "dz", "dh0")}
    sub.update({k: g[k][chans] for k in ("dD", "ddt_bias")})
    if x.nheads:
        sub["dA"] = g["dA"][[0, x.nheads - 1]]
        r["dA"] = r["dA"].reshape(2, hd * x.N).sum(axis=1)
    else:
        sub["dA"] = g["dA"][chans]
    check(x, sub, r, f"workload {index} channels={len(chans)}")
    # identities at full size
    y = run_gpu(_as_f32(x)).astype(np.float64)
    dot = lambda a, b: float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))
    loss = dot(dy, y)
    scale = float(np.sum(np.abs(np.asarray(dy, np.float64) * y)))
    via_c = dot(g["dC"], x.C) + dot(g["dD"], x.D)
    via_b = dot(g["dB"], x.B) + dot(g["dD"], x.D)
    via_u = dot(g["du"], x.u)
    print(f"loss={loss:.6e} via_C={via_c:.6e} via_B={via_b:.6e} via_u={via_u:.6e} scale={scale:.3e}", flush=True)
    assert abs(via_c - loss) <= 1e-4 * scale
    assert abs(via_b - loss) <= 1e-4 * scale
    # du is rounded to bf16: each element within 2^-9 of its value
    assert abs(via_u - loss) <= 2e-3 * float(np.sum(np.abs(np.asarray(g["du"], np.float64) * x.u))) + 1e-4 * scale
    torch.cuda.synchronize()


def test_backward_split_sequence_chain_rule():
    """Backward of two halves, the second started from the forward's state at the cut
    and its dh0 fed to the first as dh_last, equals one backward over the whole."""
    import torch
    import selective_state_space_79_amd as ssm
    from selective_state_space_79_amd.inputs import to_device, io_to_device

    announce("bwd split chain rule (2, 1024, 128, 16) f32")
    x = make_inputs(2, 1024, 128, 16, seed=77, io="f32")
    dy, dhl = make_cotangents(x, seed=78, with_dh_last=True)
    dev = to_device(x)
    dyd = io_to_device(x, dy)
    dhd = torch.from_numpy(dhl).cuda()
    full = ssm.selective_scan_bwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                                  dev["dt_bias"], dy=dyd, dh_last=dhd)
    s = 400
    part = lambda t, a, b: t[..., a:b].contiguous()
    _, hs = ssm.selective_scan_fwd(part(dev["u"], 0, s), part(dev["delta"], 0, s), dev["A"], part(dev["B"], 0, s),
                                   part(dev["C"], 0, s), dev["D"], part(dev["z"], 0, s), dev["dt_bias"],
                                   return_state=True)
    g2 = ssm.selective_scan_bwd(part(dev["u"], s, None), part(dev["delta"], s, None), dev["A"],
                                part(dev["B"], s, None), part(dev["C"], s, None), dev["D"], part(dev["z"], s, None),
                                dev["dt_bias"], dy=part(dyd, s, None), h0=hs, dh_last=dhd)
    g1 = ssm.selective_scan_bwd(part(dev["u"], 0, s), part(dev["delta"], 0, s), dev["A"], part(dev["B"], 0, s),
                                part(dev["C"], 0, s), dev["D"], part(dev["z"], 0, s), dev["dt_bias"],
                                dy=part(dyd, 0, s), dh_last=g2["dh0"])
    torch.cuda.synchronize()
    n = lambda t: t.double().cpu().numpy()
    for k in ("du", "ddelta", "dz", "dB", "dC"):
        cat = np.concatenate([n(g1[k]), n(g2[k])], axis=-1)
        assert np.max(np.abs(cat - n(full[k]))) <= 1e-4 * max(1.0, np.max(np.abs(n(full[k])))), k
    for k in ("dA", "dD", "ddt_bias"):
        assert np.max(np.abs(n(g1[k]) + n(g2[k]) - n(full[k]))) <= 1e-4 * max(1.0, np.max(np.abs(n(full[k])))), k
    assert np.max(np.abs(n(g1["dh0"]) - n(full["dh0"]))) <= 1e-4 * max(1.0, np.max(np.abs(n(full["dh0"]))))


def test_backward_worked_example():
    """The qubittool scalar example (retain/write/read) as a one-state scan: the
    gradient of the summed outputs with respect to each value is the sum of the reads
    that see it, weighted by the retains in between (write 1, 0, 1; retain .1, .95,
    .5; read 1): d/dvalue_0 = 1 + .95 + .95*.5, d/dvalue_1 = 0, d/dvalue_2 = 1."""
    import math
    import torch
    import selective_state_space_79_amd as ssm

    announce("bwd worked example")
    retain = np.array([0.10, 0.95, 0.50])
    write = np.array([1.0, 0.0, 1.0])
    dt = -np.log(retain)
    f = lambda a: torch.tensor(np.asarray(a, np.float32).reshape(1, 1, 3)).cuda()
    g = ssm.selective_scan_bwd(f([2.0, 9.0, 1.0]), f([math.log(math.expm1(v)) for v in dt]),
                               torch.tensor([[-1.0]]).cuda(), f(write / dt), f(np.ones(3)), dy=f(np.ones(3)))
    torch.cuda.synchronize()
    np.testing.assert_allclose(g["du"].cpu().numpy().ravel(), [1 + 0.95 + 0.95 * 0.5, 0.0, 1.0], rtol=0, atol=2e-6)
